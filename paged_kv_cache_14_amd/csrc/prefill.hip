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
// table: two tiles in flight in registers, two stages in LDS, K and V
// row-major in padded rows.
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
constexpr int kCascadeWorkgroups = 512;  // 2 per compute unit
constexpr int kPrefillWgsPerXcd = 64;    // 2 per compute unit of an XCD
constexpr int kWaveRows = 32;   // query rows per wave

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
  int32_t num_pairs;        // sequences x KV heads
  int32_t per_xcd;          // items per XCD queue
  const int32_t* order;     // sequences by decreasing prefill work
  int32_t* queue;           // [8] next item of each XCD queue (0 at launch)
  float scale_log2;
  // Shared-prefix pass only: the plan's work items and their count, and the
  // records [S][Hkv][G][kPrefixChunks][kRecFloats].
  const int32_t* items;
  const int32_t* count;
  int32_t max_items;
  float* prefix_rec;
};

// Accumulator row i of the 32x32 S^T product holds key perm(i) of a 32-key
// half (bits 2 and 3 of i swapped).  Lane l then owns keys 8*(l/32) .. +7 and
// 16 + 8*(l/32) .. +7 of the half: for each 16-key step of P.V, exactly the
// 8 keys its B operand needs.
__device__ inline int key_perm(int i) { return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1); }
// LDS rows are padded so the lanes one LDS cycle serves hit distinct banks,
// and every operand address is one per-lane base plus an immediate offset.
// K: key k is stored at row key_perm(k) (the permutation is its own
// inverse), so the S^T operand reads rows 0..31 in lane order; a 272-B row
// stride (17 x 16 B) puts consecutive rows in consecutive 16-B bank groups.
// V: row = key, 288-B stride (18 x 16 B): the transposing reads of 4
// consecutive keys x 32 B land in 8 distinct 16-B bank groups.
constexpr int kRowK = 136;  // elements per K row in LDS (128 + 8 padding)
constexpr int kRowV = 144;  // elements per V row in LDS (128 + 16 padding)

template <int S> struct Stage { static constexpr int value = S; };

// ---- Shared-prefix groups ---------------------------------------------------
// Sequence x may join a group when it has exactly one query token.  Of its
// blocks, only full blocks before the one holding its last key are shared
// work, so the decode kernel always has at least one block left to finish.
struct PlanArgs {
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* qsl;
  int32_t* starts;   // [S][2]
  int32_t* items;    // [max_items][8]: lead, shared, q0, members, chunk, chunks, g, -
  int32_t* count;    // items written (the decode kernel resets it to 0)
  int32_t max_blocks;
  int32_t max_context_len;
  int32_t num_seqs;
  int32_t G;
  int32_t Hkv;
  int32_t max_items;
};

__device__ inline int shareable_blocks(const PlanArgs& a, int x) {
  // never past the table row, nor past the caller's bound on context lengths
  return min((a.context_lens[x] - 1) / kBlockSize,
             min(a.max_blocks - 1, (a.max_context_len - 1) / kBlockSize));
}
// A link joins x to x-1: both one-token sequences, both with at least
// kCascadeMinBlocks shareable blocks, and the same first kCascadeMinBlocks
// physical blocks in their tables.  Every load is issued unconditionally
// (planning only runs when table rows hold more than kCascadeMinBlocks
// entries), so the test costs one memory round trip.
__device__ inline bool linked(const PlanArgs& a, int x) {
  if (x < 1 || x >= a.num_seqs) return false;
  const int32_t* t1 = a.block_tables + (size_t)x * a.max_blocks;
  const int32_t* t0 = t1 - a.max_blocks;
  bool eq = true;
#pragma unroll
  for (int i = 0; i < kCascadeMinBlocks; ++i) eq &= t1[i] == t0[i];
  const int q0 = a.qsl[x - 1], q1 = a.qsl[x], q2 = a.qsl[x + 1];
  return eq && q2 - q1 == 1 && q1 - q0 == 1 && shareable_blocks(a, x) >= kCascadeMinBlocks &&
         shareable_blocks(a, x - 1) >= kCascadeMinBlocks;
}

// One wave per sequence s.  Groups are maximal runs of links cut every
// `max_members` sequences, so every wave derives the same groups from the
// same tables.  A sequence in no group gets starts (0, 0).  A group's lead
// finds the blocks all members share, writes every member's starts entry
// (shared blocks, chunks) and appends one work item per (chunk, KV head).
__global__ __launch_bounds__(256) void cascade_plan_kernel(PlanArgs a) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= a.num_seqs) return;
  const int max_members = min(kCascadeMaxMembers, kWgRows / a.G);  // <= 32
  // Lane i examines sequence x = s + 32 - i: bit 32 + k of `links` is the
  // link into s - k, bit 32 - d the link into s + d.  A group has at most 32
  // members, so all of s's group lies in these 64 sequences.
  const int x = s + 32 - lane;
  const bool in = x >= 0 && x < a.num_seqs;
  const uint64_t links = __builtin_amdgcn_ballot_w64(linked(a, x));
  const int shr = in ? shareable_blocks(a, x) : 0;
  const int qs = in ? a.qsl[x] : 0;
  const uint32_t back = (uint32_t)(links >> 32);  // bit k: link into s - k
  int run;                                        // consecutive links ending at s
  if (~back) {
    run = __builtin_ctz(~back);
  } else {  // a run longer than 32 sequences: keep counting backwards
    run = 32;
    for (int base = s - 32;; base -= 64) {
      const uint64_t m2 = ~__builtin_amdgcn_ballot_w64(linked(a, base - lane));
      if (m2) {
        run += __builtin_ctzll(m2);
        break;
      }
      run += 64;
    }
  }
  const int j = run % max_members;
  // Links into s+1, s+2, ... as bits 0, 1, ...
  const uint32_t fwd = __builtin_bitreverse32((uint32_t)links);
  const int ahead = ~fwd ? (int)__builtin_ctz(~fwd) : 32;
  const int members = j + 1 + min(ahead, max_members - 1 - j);
  if (members == 1) {
    if (lane == 0) {
      a.starts[2 * s] = 0;
      a.starts[2 * s + 1] = 0;
    }
    return;
  }
  if (j != 0) return;  // the lead plans the group
  const int lead = s;
  // Member m is lane 32 - m.
  int cap = (lane <= 32 && lane > 32 - members) ? shr : INT32_MAX;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) cap = min(cap, __shfl_xor(cap, o));
  const int q0 = __shfl(qs, 32);
  // Shared blocks: the members' common table prefix, at most `cap`.  Each
  // lane compares (member, block) pairs with the previous member's row, 8
  // pairs per round trip (a repeated last pair is harmless).
  int first_diff = cap;
  const int pairs = (members - 1) * cap;
  const int32_t* tab1 = a.block_tables + (size_t)(lead + 1) * a.max_blocks;
  for (int i0 = 0; i0 < pairs; i0 += 8 * 64) {
    int v1[8], v0[8], bk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = min(i0 + k * 64 + lane, pairs - 1);
      const int xm = i / cap;
      bk[k] = i - xm * cap;
      const int32_t* t1 = tab1 + (size_t)xm * a.max_blocks + bk[k];
      v1[k] = t1[0];
      v0[k] = t1[-a.max_blocks];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (v1[k] != v0[k]) first_diff = min(first_diff, bk[k]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) first_diff = min(first_diff, __shfl_xor(first_diff, o));
  const int shared = first_diff;  // >= kCascadeMinBlocks: the links compared those
  // Chunks of at least kChunkTiles tiles (when there are that many), at most
  // kPrefixChunks, each one workgroup per KV head.
  const int tiles = (shared * kBlockSize + kTileKeys - 1) / kTileKeys;
  const int chunks = min(kPrefixChunks, max(1, tiles / kChunkTiles));
  if (lane < members) {
    a.starts[2 * (lead + lane)] = shared;
    a.starts[2 * (lead + lane) + 1] = chunks;
  }
  const int n_items = chunks * a.Hkv;
  int slot = 0;
  if (lane == 0) slot = atomicAdd(a.count, n_items);
  slot = __shfl(slot, 0);
  for (int i = lane; i < n_items; i += 64) {
    if (slot + i >= a.max_items) break;  // only if the caller's bounds were wrong
    int32_t* it = a.items + (size_t)(slot + i) * 8;
    const int c = i / a.Hkv;
    *reinterpret_cast<int4*>(it) = int4{lead, shared, q0, members};
    *reinterpret_cast<int4*>(it + 4) = int4{c, chunks, i - c * a.Hkv, 0};
  }
}

// kCascade == false: prefill.  A workgroup owns 128 (token, head) rows of one
// sequence and KV head, under the bottom-right causal mask.
// kCascade == true: shared-prefix pass for decode.  A workgroup takes one
// work item of the plan (group, chunk, KV head): it attends the (token, head)
// rows of all the group's members (at most 128) to the chunk's keys of the
// shared blocks, with no mask (every member sees them all), and writes each
// row's (max, sum, unnormalised output) record, which the decode kernel
// merges with the member's own tail.
typedef uint16_t KTiles[2][kTileKeys * kRowK];
typedef uint16_t VTiles[2][kTileKeys * kRowV];

// One work unit: prefill work item `item` (kCascade false) or shared-prefix
// work item `item` of the plan.  Returns early when the unit
// has nothing to do; ends with every LDS read done (the last tile step ends
// on a barrier).
template <typename T, bool kCascade>
__device__ __forceinline__ void attend(const PrefillArgs& a, int item, KTiles& k_lds,
                                       VTiles& v_lds) {
  using MM = Mfma<T>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, lrow = lane & 31;

  int s, g, q0, n, rows, r0, C, N, t_begin = 0, chunk = 0;
  if constexpr (!kCascade) {
    // Work item k of XCD x's queue (item = 8k + x).  (sequence, KV head)
    // pairs are dealt round-robin to the 8 XCDs, sequences in order of
    // decreasing prefill work, so the longest items start first and every
    // XCD gets a share of long and short ones.  The query tiles of a pair are
    // adjacent in the queue, so they run at about the same time on the same
    // XCD and share its L2 while streaming the same K/V; a head's heavier
    // (later) tiles come first.
    const int k = item >> 3;
    const int pair = (item & 7) + 8 * (k / a.tiles_per_head);
    if (pair >= a.num_pairs) return;
    const int rank = pair / a.Hkv;
    s = a.order[rank];
    g = pair - rank * a.Hkv;
    const int tile = a.tiles_per_head - 1 - (k - (k / a.tiles_per_head) * a.tiles_per_head);
    q0 = a.qsl[s];
    n = a.qsl[s + 1] - q0;
    rows = n * a.G;
    if (rows <= kDecodeRows) return;  // short runs belong to the decode kernel
    r0 = tile * kWgRows;
    if (r0 >= rows) return;
    C = a.context_lens[s];
    N = min((C + kBlockSize - 1) / kBlockSize, a.max_blocks);  // never past the table row
  } else {
    const int4 i0 = *reinterpret_cast<const int4*>(a.items + (size_t)item * 8);
    const int4 i1 = *reinterpret_cast<const int4*>(a.items + (size_t)item * 8 + 4);
    s = i0.x;  // the lead: its table row is the group's
    const int shared = i0.y;
    q0 = i0.z;
    rows = i0.w * a.G;  // members * G
    chunk = i1.x;
    const int chunks = i1.y;
    g = i1.z;
    n = 1;
    r0 = 0;
    const int tiles = (shared * kBlockSize + kTileKeys - 1) / kTileKeys;
    t_begin = chunk * tiles / chunks;
    // Keys [t_begin*64, C) of the shared range, all visible to every row.
    C = min((chunk + 1) * tiles / chunks * kTileKeys, shared * kBlockSize);
    N = shared;
  }

  const int my_row = r0 + wave * kWaveRows + lrow;
  const bool row_ok = my_row < rows;
  const int row_c = row_ok ? my_row : rows - 1;  // padding rows mirror the last real row
  // Prefill: row = token * G + head.  Cascade: row = member * G + head, and
  // member m's one token is query row qsl[s + m] (= q0 + m for decode).
  const int tok = row_c / a.G;
  const int hg = row_c - tok * a.G;
  const int lim = kCascade ? C - 1 : C - n + tok;  // last key this row sees
  const int tok_first = r0 / a.G;
  const int tok_last = min(rows - 1, r0 + kWgRows - 1) / a.G;
  const int kv_end = kCascade ? C : C - n + tok_last + 1;       // keys the workgroup touches
  const int full_end = kCascade ? C : C - n + tok_first + 1;    // keys every row sees
  const int n_tiles = (kv_end + kTileKeys - 1) / kTileKeys;
  const bool wave_live = r0 + wave * kWaveRows < rows;

  // Q^T as the B operand: lane l holds dims 16*kk + 8*h .. +7 of row l%32.
  u32x4 qreg[8];
  {
    const uint16_t* qrow = a.q + ((size_t)(q0 + tok) * a.Hq + g * a.G + hg) * kHeadDim + h * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qreg[kk] = load16(qrow + kk * 16);
  }

  const int32_t* tab = a.block_tables + (size_t)s * a.max_blocks;
  // Block base addresses are uniform (scalar 64-bit arithmetic); each lane
  // adds a 32-bit byte offset, so the loads use scalar-base addressing.
  const size_t blk_bytes = (size_t)a.Hkv * kBlockSize * kHeadDim * sizeof(uint16_t);
  const char* k_base = reinterpret_cast<const char*>(a.k_pool) +
                       (size_t)g * kBlockSize * kHeadDim * sizeof(uint16_t);
  const char* v_base = reinterpret_cast<const char*>(a.v_pool) +
                       (size_t)g * kBlockSize * kHeadDim * sizeof(uint16_t);
  const uint32_t lane_bytes = ((tid >> 4) * kHeadDim + (tid & 15) * 8) * sizeof(uint16_t);
  // Loader: thread t moves 16-B chunk t%16 of token t/16 of each of the
  // tile's 4 blocks, for K and for V (coalesced 1 KiB per wave per block).
  // Block indices are clamped to the sequence's last block: the extra keys of
  // the final tile are masked, and their V rows are stored as zeros.
  const int my_key = tid >> 4, my_chunk = tid & 15;
  int ids[4];
  auto fetch_ids = [&](int t, int (&out)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = tab[min(t * 4 + i, N - 1)];
  };
  // Two register sets: while tile t is consumed from LDS, tile t+1 waits in
  // one set and tile t+2 is loading into the other (two tiles in flight).
  u32x4 kreg[2][4], vreg[2][4];
  auto load_tile = [&](int set, const int (&id)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t blk = (size_t)id[i] * blk_bytes;
      constexpr int32_t kTileBytes = kBlockSize * kHeadDim * sizeof(uint16_t);
      kreg[set][i] = load16_at(k_base + blk, lane_bytes, kTileBytes);
      vreg[set][i] = load16_at(v_base + blk, lane_bytes, kTileBytes);
    }
  };
  // Writer addresses (elements), per 16-key group i of the tile: K row
  // key_perm(key), V row key.
  const int k_w = key_perm(my_key) * kRowK + my_chunk * 8;
  const int v_w = my_key * kRowV + my_chunk * 8;
  auto store_tile = [&](int st, int set, int t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) store16(&k_lds[st][k_w + 16 * i * kRowK], kreg[set][i]);
    if ((t + 1) * kTileKeys > C) {  // last tile: slots past C may hold NaN, store 0
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v =
            t * kTileKeys + my_key + 16 * i < C ? vreg[set][i] : u32x4{0u, 0u, 0u, 0u};
        store16(&v_lds[st][v_w + 16 * i * kRowV], v);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) store16(&v_lds[st][v_w + 16 * i * kRowV], vreg[set][i]);
    }
  };

  // Reader bases (elements).  S^T operand (half kt, 16-dim step kk): row
  // kt*32 + l%32, dims 16*kk + 8*h .. +7.  V^T operand (dim tile dt, 16-key
  // step ks, half r): lane j of 16-lane group q = l/16 reads key
  // ks*16 + (q/2)*8 + 4r + j/4, dims dt*32 + (q%2)*16 + 4*(j%4) .. +3.
  const int q16 = lane >> 4, j16 = lane & 15;
  const int k_r = lrow * kRowK + h * 8;
  const int v_r = ((q16 >> 1) * 8 + (j16 >> 2)) * kRowV + (q16 & 1) * 16 + 4 * (j16 & 3);

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  // Running max in raw logit units; the weights are 2^(s*c - m_ref*c) <= 2^8.
  float m_ref = kNegBig, l = 0.f;
  const float c = a.scale_log2;

  fetch_ids(t_begin, ids);
  load_tile(0, ids);
  store_tile(0, 0, t_begin);  // waits for Q and the first tile
  fetch_ids(t_begin + 1, ids);
  load_tile(1, ids);          // the second tile stays in flight into the loop
  fetch_ids(t_begin + 2, ids);
  __syncthreads();

  // One tile step; the stage is a compile-time constant so every LDS address
  // below is a per-lane base plus an immediate offset.
  auto step = [&](const int t, auto stage) {
    constexpr int st = decltype(stage)::value;
    // Loads and stores are unconditional (tiles past the end re-read the last
    // block and land in a stage nobody reads), so every path through the loop
    // has the same loads outstanding and the wait counts stay exact.
    int ids_next[4];
    load_tile(st, ids);  // tile t+2 into the set tile t came through
    fetch_ids(t + 3, ids_next);

    if (wave_live) {
      const uint16_t* kl = k_lds[st];
      const uint16_t* vl = v_lds[st];
      // S^T for the two 32-key halves of the tile (independent chains, interleaved).
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          sacc[kt] = MM::mm32(*reinterpret_cast<const u32x4*>(kl + k_r + kt * 32 * kRowK + kk * 16),
                              qreg[kk], sacc[kt]);
      // Causal mask (only tiles reaching past the keys every row sees).
      if ((t + 1) * kTileKeys > full_end) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = t * kTileKeys + kt * 32 + (v >> 3) * 16 + h * 8 + (v & 7);
            sacc[kt][v] = key <= lim ? sacc[kt][v] : -__builtin_inff();
          }
      }
      // Row max over the lane's 32 logits as a tree of 3-input maxima.
      float m3[11];
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        const int a = 3 * i, b = 3 * i + 1, d = 3 * i + 2;
        m3[i] = fmaxf(fmaxf(sacc[a >> 4][a & 15], sacc[b >> 4][b & 15]), sacc[d >> 4][d & 15]);
      }
      m3[10] = fmaxf(sacc[1][14], sacc[1][15]);
      float mt = fmaxf(fmaxf(m3[0], m3[1]), m3[2]);
      mt = fmaxf(fmaxf(mt, m3[3]), m3[4]);
      mt = fmaxf(fmaxf(mt, m3[5]), m3[6]);
      mt = fmaxf(fmaxf(mt, m3[7]), m3[8]);
      mt = fmaxf(fmaxf(mt, m3[9]), m3[10]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      // Move the reference max only when some row's max grew by more than
      // 2^8 in weight: the rescale of O is then rare after the first tile.
      if (__builtin_amdgcn_ballot_w64((mt - m_ref) * c > 8.f)) {
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = fast_exp2((m_ref - m_new) * c);
        m_ref = m_new;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      }
      const float mc = m_ref * c;
      u32x4 pb[4], pl[4];  // the weights as hi + lo pairs of the input type (split_weights)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p0 = fast_exp2(__builtin_fmaf(sacc[kt][2 * e], c, -mc));
          const float p1 = fast_exp2(__builtin_fmaf(sacc[kt][2 * e + 1], c, -mc));
          const u32x2 w = split_weights<T>(p0, p1);
          pb[kt * 2 + (e >> 2)][e & 3] = w[0];
          pl[kt * 2 + (e >> 2)][e & 3] = w[1];
          l += p0 + p1;
        }

      // O^T += V^T P^T with V^T read transposed out of row-major LDS, for the
      // weights' hi and lo parts; the four dim tiles are independent chains,
      // interleaved.
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const uint16_t* vp = vl + v_r + ks * 16 * kRowV + dt * 32;
          const u32x2 lo = ds_read_tr(vp);
          const u32x2 hi = ds_read_tr(vp + 4 * kRowV);
          const u32x4 vop = {lo[0], lo[1], hi[0], hi[1]};
          o[dt] = MM::mm32(vop, pb[ks], o[dt]);
          o[dt] = MM::mm32(vop, pl[ks], o[dt]);
        }
    }

    store_tile(st ^ 1, st ^ 1, t + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) ids[i] = ids_next[i];
    __syncthreads();
  };

  int t = t_begin;
  for (; t + 1 < n_tiles; t += 2) {
    step(t, Stage<0>{});
    step(t + 1, Stage<1>{});
  }
  if (t < n_tiles) step(t, Stage<0>{});

  // Normalise and store: lane l holds dims dt*32 + 8*(v/4) + 4*h + v%4.
  const float lt = l + __shfl_xor(l, 32);
  if constexpr (kCascade) {
    // Record of row (member tok, head hg) for this chunk: the running max in
    // base-2 units, the sum of weights and the unnormalised output.
    if (row_ok) {
      float* rec = a.prefix_rec +
                   ((((size_t)(s + tok) * a.Hkv + g) * a.G + hg) * kPrefixChunks + chunk) *
                       kRecFloats;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(rec + dt * 32 + q4 * 8 + h * 4) =
              f32x4{o[dt][q4 * 4 + 0], o[dt][q4 * 4 + 1], o[dt][q4 * 4 + 2], o[dt][q4 * 4 + 3]};
      if (h == 0) {
        rec[128] = lt > 0.f ? m_ref * c : kNegBig;  // an empty chunk weighs nothing
        rec[129] = lt;
      }
    }
    return;
  }
  if (row_ok) {
    const float inv = 1.f / lt;
    uint16_t* orow = a.out + ((size_t)(q0 + tok) * a.Hq + g * a.G + hg) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 pk;
        pk[0] = Pair<T>::pack(o[dt][q4 * 4 + 0] * inv, o[dt][q4 * 4 + 1] * inv);
        pk[1] = Pair<T>::pack(o[dt][q4 * 4 + 2] * inv, o[dt][q4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + dt * 32 + q4 * 8 + h * 4) = pk;
      }
    }
  }
}

// The read-only index arrays come again as __restrict__ parameters: the
// compiler may then prove that no store of the kernel (outputs, records,
// queue atomics) reaches them, and keep their wave-uniform loads on the
// scalar unit even in the persistent loop.  (As vector loads they would share
// the in-order vector-memory counter with the tile prefetch, and waiting for
// a block id would wait for the tiles issued before it.)
template <typename T, bool kCascade>
__global__ __launch_bounds__(256, 2) void prefill_kernel(
    PrefillArgs args, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ order_or_items) {
  __shared__ __attribute__((aligned(16))) KTiles k_lds;
  __shared__ __attribute__((aligned(16))) VTiles v_lds;
  PrefillArgs a = args;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.qsl = qsl;
  if constexpr (kCascade)
    a.items = order_or_items;
  else
    a.order = order_or_items;
  if constexpr (kCascade) {
    // Persistent: workgroups take the plan's items in turn.
    const int count = min(*a.count, a.max_items);
    for (int item = blockIdx.x; item < count; item += gridDim.x) {
      attend<T, true>(a, item, k_lds, v_lds);
      __syncthreads();
    }
  } else {
    // Persistent: the workgroups of XCD x (workgroup b runs on XCD b % 8) take
    // the items of that XCD's queue in turn, so a workgroup that finishes a
    // short item starts the next one at once, whatever the others do.
    __shared__ int next;
    const int x = blockIdx.x & 7;
    for (;;) {
      if (threadIdx.x == 0) next = atomicAdd(a.queue + x, 1);
      __syncthreads();
      // Uniform by construction; saying so keeps everything derived from it
      // (sequence, table row, block ids) in scalar registers and loads.
      const int k = __builtin_amdgcn_readfirstlane(next);
      __syncthreads();  // all have read `next` before it is taken again
      if (k >= a.per_xcd) break;
      attend<T, false>(a, k * 8 + x, k_lds, v_lds);
      __syncthreads();
    }
  }
}

// ---- Wide prefill: 256-row workgroups, tiles loaded straight into LDS ----
//
// For calls whose sequences bring many query rows per KV head (long prompt
// chunks, large GQA groups, multi-turn runs of more than 128 rows).  A
// workgroup (one per compute unit) owns 256 rows of one (sequence, KV head).
// 4-wave form (one wave per SIMD), for calls of 1024 rows or more: each wave
// owns 64 rows as two 32-row halves, so every K or V operand it reads from
// LDS feeds two matrix-core products (half the LDS reads per flop of the
// 32-row waves above).  8-wave form (two waves per SIMD), for calls of
// 129..1023 rows: 32 rows per wave, so that a run of up to 256 rows reads its
// K/V once without padding rows to 64.  Tiles of 64 keys travel HBM -> LDS
// through the buffer loads' LDS mode, without staging registers, into four
// stages: while a wave works on tiles t and t+1, tiles t+2 and t+3 are in
// flight.  The work runs in 32-key sub-tiles j: one step computes
// S(j+2) = K(j+2) Q^T, the weights of j+1 and O += V(j)^T P(j)^T, three
// independent pieces, so the products and the softmax's vector work
// interleave within a wave.
//
// LDS rows are 256 B, unpadded (a load writes 1 KiB contiguously, 16 B per
// lane); the 16-B chunks of a row are XOR-swizzled so that the lanes one LDS
// cycle serves hit distinct banks:
//   K: row R holds key key_perm(R); position p holds chunk p ^ (R & 15),
//   V: row k holds key k; position p holds chunk p ^ v_swizzle(k & 3).
constexpr int kRoundedMinKeys = 1024; // keys every row of an item sees, from which weights may be rounded
constexpr int kWideWgsPerXcd = 32;    // one per compute unit of an XCD
constexpr int64_t kWideMinRows = 1024;  // rows per KV head from which a call takes the 4-wave form
constexpr int kTileBytes = kTileKeys * kHeadDim * (int)sizeof(uint16_t);   // one K or V tile
constexpr int kSlabBytes = kBlockSize * kHeadDim * (int)sizeof(uint16_t);  // one block, one head
constexpr int kRowBytes = kHeadDim * (int)sizeof(uint16_t);

typedef __attribute__((address_space(3))) void lds_void;

// Transposing V reads take 4 consecutive keys x 4 chunks per 16-lane pair;
// this swizzle sends the 16 (key, chunk) pairs to 16 distinct 16-B bank
// groups, and any 8 of them with the same chunk parity to 8 distinct ones.
__device__ inline int v_swizzle(int k) { return 10 * (k & 1) + 4 * ((k >> 1) & 1); }

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Workgroup barrier of the tile pipeline.  Waits for this wave's LDS and
// scalar accesses only: the tile loads in flight stay in flight (a plain
// __syncthreads would wait for them too).
__device__ inline void pipeline_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

typedef uint16_t WideTile[kTileBytes / sizeof(uint16_t)];
// A pipeline stage is one K tile and one V tile, each its own LDS array (the
// compiler then waits, before an LDS read, only for the tile loads into that
// array).  The four V tiles take the low 64 KiB and the K tiles the next 64
// KiB, so every V read's offset from a lane's base fits the 16-bit offset
// field of the LDS instructions, and the K reads' from one base past them.

// S^T products for the wide kernel, written out so that the scores land in
// vector registers, where the softmax reads them, while O accumulates in the
// accumulation registers (the compiler gives all of a kernel's products one
// form, and every score would then cost a register copy).  Q, the B operand,
// lives in the accumulation registers.  The compiler does not see these as
// matrix-core products, so a vector read of the result must first pass
// settle_scores(), which provides the wait states the hardware needs between
// a product writing a vector register and a vector instruction reading it.
template <typename T> struct MfmaScores;
template <> struct MfmaScores<bf16> {
  __device__ static inline f32x16 first(u32x4 a, u32x4 b) {
    f32x16 d;
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
    return d;
  }
  __device__ static inline void next(f32x16& d, u32x4 a, u32x4 b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
  }
};
template <> struct MfmaScores<f16> {
  __device__ static inline f32x16 first(u32x4 a, u32x4 b) {
    f32x16 d;
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
    return d;
  }
  __device__ static inline void next(f32x16& d, u32x4 a, u32x4 b) {
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
  }
};
// 21 wait states, ordered before every read of the scores: a vector read of
// a product's result needs the product's passes + 4 on gfx950, 20 for a
// 16-pass product.
template <int H>
__device__ inline void settle_scores(f32x16 (&s)[H]) {
  if constexpr (H == 2)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(s[0]), "+v"(s[1]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(s[0]));
}

// Calls f(Stage<I>{}) for I = B .. E-1, in order.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Stage<B>{});
    static_for<B + 1, E>(f);
  }
}

// Max and sum of a value with the one lane l ^ 32 holds (v_permlane32_swap
// exchanges the two 32-lane halves of a pair of registers; no LDS access).
__device__ inline float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One wide work item; returns early (before any tile load) when it has no
// rows, and otherwise ends with every tile load landed and every LDS read done.
// kHalves 2: 4 waves of 64 rows; kHalves 1: 8 waves of 32 rows, and waves
// without real rows skip the products (they still load their share).
template <typename T, int kHalves>
__device__ __forceinline__ void attend_wide(const PrefillArgs& a, int item, WideTile& k0,
                                            WideTile& k1, WideTile& k2, WideTile& k3, WideTile& v0,
                                            WideTile& v1, WideTile& v2, WideTile& v3) {
  using MM = Mfma<T>;
  constexpr int kWaves = 8 / kHalves;
  constexpr int kThreads = 64 * kWaves;
  constexpr int kRowsPerWave = 32 * kHalves;
  // Tile loads per wave and tile, and the block-id load that goes with them.
  constexpr int kLoads = kWaves == 4 ? 8 : 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blk = wave & 3;  // the block of a tile this wave loads
  const int h = lane >> 5, lrow = lane & 31;

  // Work item k of XCD x's queue, as for the narrow kernel, with 256-row tiles.
  const int k = item >> 3;
  const int pair = (item & 7) + 8 * (k / a.tiles_per_head);
  if (pair >= a.num_pairs) return;
  const int rank = pair / a.Hkv;
  const int s = a.order[rank];
  const int g = pair - rank * a.Hkv;
  const int tile = a.tiles_per_head - 1 - (k - (k / a.tiles_per_head) * a.tiles_per_head);
  const int q0 = a.qsl[s];
  const int n = a.qsl[s + 1] - q0;
  const int rows = n * a.G;
  if (rows <= kDecodeRows) return;  // short runs belong to the decode kernel
  const int r0 = tile * kWideWgRows;
  if (r0 >= rows) return;
  const int C = a.context_lens[s];
  const int N = min((C + kBlockSize - 1) / kBlockSize, a.max_blocks);  // never past the table row

  // The lane's row in each half hh: r0 + 32*(kHalves*wave + hh) + lane%32.
  // Padding rows mirror the last real row.
  int lim[kHalves], tok[kHalves], hg[kHalves];
  bool row_ok[kHalves];
  u32x4 qreg[kHalves][8];
#pragma unroll
  for (int hh = 0; hh < kHalves; ++hh) {
    const int my_row = r0 + wave * kRowsPerWave + hh * 32 + lrow;
    row_ok[hh] = my_row < rows;
    const int row_c = row_ok[hh] ? my_row : rows - 1;
    tok[hh] = row_c / a.G;
    hg[hh] = row_c - tok[hh] * a.G;
    lim[hh] = C - n + tok[hh];
    const uint16_t* qrow =
        a.q + ((size_t)(q0 + tok[hh]) * a.Hq + g * a.G + hg[hh]) * kHeadDim + h * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qreg[hh][kk] = load16(qrow + kk * 16);
  }

  const int tok_first = r0 / a.G;
  const int tok_last = min(rows - 1, r0 + kWideWgRows - 1) / a.G;
  const int kv_end = C - n + tok_last + 1;     // keys the workgroup touches
  const int full_end = C - n + tok_first + 1;  // keys every row sees
  const int n_tiles = (kv_end + kTileKeys - 1) / kTileKeys;
  const bool wave_live = r0 + wave * kRowsPerWave < rows;
  const bool compute = kHalves == 2 || wave_live;

  // Tile loads: with 4 waves, wave w moves block w of the tile (16 keys), K
  // and V; with 8, wave w moves block w%4 of K (w < 4) or of V.  A block is
  // four 1-KiB loads; lane j of a load fills LDS bytes 16j .. 16j+15 of it,
  // i.e. row 4i + j/16 of the block's 16, swizzled position j%16.
  const int32_t* tab = a.block_tables + (size_t)s * a.max_blocks;
  const size_t blk_bytes = (size_t)a.Hkv * kSlabBytes;
  const char* k_base = reinterpret_cast<const char*>(a.k_pool) + (size_t)g * kSlabBytes;
  const char* v_base = reinterpret_cast<const char*>(a.v_pool) + (size_t)g * kSlabBytes;
  const int lr = lane >> 4, lp = lane & 15;
  uint32_t k_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int R = 4 * i + lr;  // LDS row within the block (R & 15 == R)
    k_src[i] = key_perm(R) * kRowBytes + ((lp ^ R) << 4);
  }
  const uint32_t v_src = lr * kRowBytes + ((lp ^ v_swizzle(lr)) << 4);
  // Block ids of later tiles come through vector loads, two steps ahead, so
  // they share the in-order count of the tile loads (a scalar load in flight
  // would make the compiler wait for everything before each LDS read).  In
  // the 8-wave form the compiler still waits for each step's id before the
  // step's loads; taking every load out of its view to drop those waits
  // measured no faster there (its steps wait on the products instead).
  // Tiles past the end re-read the last block and land in a stage nobody
  // reads, so every step has the same loads outstanding.
  const auto tab_rsrc = buffer_rsrc(tab, a.max_blocks * (int32_t)sizeof(int32_t));
  auto load_id = [&](int t) -> int32_t {
    return __builtin_amdgcn_raw_buffer_load_b32(tab_rsrc, min(4 * t + blk, N - 1) * 4, 0, 0);
  };
  auto issue = [&](int32_t id_any_lane, WideTile& kt_lds, WideTile& vt_lds) {
    const int id = __builtin_amdgcn_readfirstlane(id_any_lane);
    const auto kr = buffer_rsrc(k_base + (size_t)id * blk_bytes, kSlabBytes);
    const auto vr = buffer_rsrc(v_base + (size_t)id * blk_bytes, kSlabBytes);
    char* kd = reinterpret_cast<char*>(kt_lds) + blk * kSlabBytes;
    char* vd = reinterpret_cast<char*>(vt_lds) + blk * kSlabBytes;
    if (kWaves == 4 || wave < 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kd + i * 1024), 16, k_src[i], 0,
                                                 0, 0);
    }
    if (kWaves == 4 || wave >= 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vd + i * 1024), 16,
                                                 v_src, i * 1024, 0, 0);
    }
  };
  // V rows of the last tile past the context may hold NaN (0 x NaN would
  // reach O): they are cleared once the tile has landed.
  auto clear_v_tail = [&](WideTile& vt_lds, int t) {
    const int first = C - t * kTileKeys;
    if (first >= kTileKeys) return;
    char* vl = reinterpret_cast<char*>(vt_lds);
    for (int i = tid; i < kTileKeys * 16; i += kThreads)
      if ((i >> 4) >= first) store16(vl + (i >> 4) * kRowBytes + (i & 15) * 16, u32x4{0u, 0u, 0u, 0u});
  };

  // LDS read offsets (bytes within a stage).  S^T operand (half kt, 16-dim
  // step kk): row kt*32 + l%32, chunk 2kk + h.  V^T operand (dim tile dt,
  // 16-key step ks, key half r): lane j of 16-lane group q reads key
  // ks*16 + (q/2)*8 + 4r + j/4, dims dt*32 + (q%2)*16 + 4(j%4) .. +3.
  uint32_t k_rd[8], v_rd[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) k_rd[kk] = lrow * kRowBytes + (((2 * kk + h) ^ (lrow & 15)) << 4);
  // The K stages lie past the first 64 KiB of LDS, out of reach of the LDS
  // instructions' 16-bit offset field.  The K reads therefore add a stage's
  // address minus kKBias as the constant and carry kKBias in the lane's
  // offset register (opaque to the compiler, so that it does not fold the
  // two back into one constant): whatever address the stage has, the sum is
  // the same, and where the stage lies past kKBias the constant fits the
  // offset field, saving one address add per read.
  constexpr uint32_t kKBias = 0x10000;
  uint32_t k_rdb[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    k_rdb[kk] = k_rd[kk] + kKBias;
    asm volatile("" : "+v"(k_rdb[kk]));
  }
  {
    const int q16 = lane >> 4, j16 = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      v_rd[dt] = ((q16 >> 1) * 8 + (j16 >> 2)) * kRowBytes +
                 (((dt * 4 + (q16 & 1) * 2 + ((j16 & 3) >> 1)) ^ v_swizzle(j16 >> 2)) << 4) +
                 8 * (j16 & 1);
  }

  f32x16 o[kHalves][4];
#pragma unroll
  for (int hh = 0; hh < kHalves; ++hh)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[hh][dt] = f32x16{};
  // Per-row reference max (raw logit units) and sum of weights; the weights
  // are 2^(s*c - m_ref*c) <= 2^8.
  float m_ref[kHalves], l[kHalves], mc[kHalves];  // mc = m_ref * c
#pragma unroll
  for (int hh = 0; hh < kHalves; ++hh) {
    m_ref[hh] = kNegBig;
    l[hh] = 0.f;
  }
  const float c = a.scale_log2;

  // The pipeline runs in 32-key sub-tiles j (tile j/2, half j%2).  One step
  // computes the scores of sub-tile j+2, the weights of sub-tile j+1 (from
  // the scores of the step before) and O += P(j) V(j): three independent
  // pieces of work, so the matrix-core products of the first and last run
  // while the vector units compute the second.
  auto scores = [&](const WideTile& kt_lds, int kt, f32x16 (&sacc)[kHalves]) {
    const char* kl = reinterpret_cast<const char*>(kt_lds) + kt * 32 * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4 kop = *reinterpret_cast<const u32x4*>(kl - kKBias + k_rdb[kk]);
#pragma unroll
      for (int hh = 0; hh < kHalves; ++hh) {
        if (kk == 0)
          sacc[hh] = MfmaScores<T>::first(kop, qreg[hh][0]);
        else
          MfmaScores<T>::next(sacc[hh], kop, qreg[hh][kk]);
      }
    }
  };
  auto mask = [&](int key0, f32x16 (&sacc)[kHalves]) {
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
      // element v holds key key0 + h*8 + (v/8)*16 + v%8
      const int d = lim[hh] - key0 - h * 8;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        sacc[hh][v] = (v >> 3) * 16 + (v & 7) <= d ? sacc[hh][v] : -__builtin_inff();
    }
  };
  // Weights of one sub-tile: each row moves its reference max only when its
  // max grew by more than 2^8 in weight; alpha takes O and l to the new
  // reference (1 when it did not move).
  auto softmax = [&](const f32x16 (&sacc)[kHalves], u32x4 (&pn)[kHalves][2],
                     u32x4 (&pnl)[kHalves][2], float (&alpha)[kHalves]) {
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
      const f32x16& sv = sacc[hh];
      float mt = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
      mt = fmaxf(fmaxf(mt, sv[3]), sv[4]);
      mt = fmaxf(fmaxf(mt, sv[5]), sv[6]);
      mt = fmaxf(fmaxf(mt, sv[7]), sv[8]);
      mt = fmaxf(fmaxf(mt, sv[9]), sv[10]);
      mt = fmaxf(fmaxf(mt, sv[11]), sv[12]);
      mt = fmaxf(fmaxf(mt, sv[13]), sv[14]);
      mt = max_xor32(fmaxf(mt, sv[15]));
      const float m_new = (mt - m_ref[hh]) * c > 8.f ? fmaxf(m_ref[hh], mt) : m_ref[hh];
      alpha[hh] = fast_exp2((m_ref[hh] - m_new) * c);
      m_ref[hh] = m_new;
      const float mc = m_new * c;
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p0 = fast_exp2(__builtin_fmaf(sv[2 * e], c, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(sv[2 * e + 1], c, -mc));
        const u32x2 w = split_weights<T>(p0, p1);
        pn[hh][e >> 2][e & 3] = w[0];
        pnl[hh][e >> 2][e & 3] = w[1];
        sum += p0 + p1;
      }
      l[hh] = l[hh] * alpha[hh] + sum;
    }
  };
  auto pv = [&](const WideTile& vt_lds, int kt, const u32x4 (&pc)[kHalves][2],
                const u32x4 (&pcl)[kHalves][2]) {
    const char* vl = reinterpret_cast<const char*>(vt_lds) + kt * 32 * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const char* vp = vl + v_rd[dt] + ks * 16 * kRowBytes;
        const u32x2 lo = ds_read_tr(reinterpret_cast<const uint16_t*>(vp));
        const u32x2 hi = ds_read_tr(reinterpret_cast<const uint16_t*>(vp + 4 * kRowBytes));
        const u32x4 vop = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int hh = 0; hh < kHalves; ++hh) {
          o[hh][dt] = MM::mm32(vop, pc[hh][ks], o[hh][dt]);
          o[hh][dt] = MM::mm32(vop, pcl[hh][ks], o[hh][dt]);
        }
      }
  };
  auto rescale = [&](const float (&alpha)[kHalves]) {
    bool moved = false;
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) moved = moved || alpha[hh] != 1.f;
    if (__builtin_amdgcn_ballot_w64(moved)) {
      // O stays in the accumulation registers: each element goes through
      // one vector register and back.  (Written out so that the compiler
      // never holds O in vector registers, which would need 128 of them.)
      // The wait states cover a matrix-core result read right after the
      // last product, and the products that read O right after the writes.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int hh = 0; hh < kHalves; ++hh)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          f32x16 v = o[hh][dt];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = v[i], tmp;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\t"
                "v_mul_f32 %1, %1, %2\n\t"
                "v_accvgpr_write_b32 %0, %1"
                : "+a"(x), "=&v"(tmp)
                : "v"(alpha[hh]));
            v[i] = x;
          }
          o[hh][dt] = v;
        }
      asm volatile("s_nop 3" ::: "memory");
    }
  };
  // One pipeline step (sub-tile j): scores of sub-tile j+2 (stage kst, half
  // kh) into `sb`, weights of sub-tile jw = j+1 from `sa`, O += P(j) V(j)
  // (stage vst, half vh), written as 16 issue slots (below).  kScores
  // false: no sub-tile j+2.
  f32x16 sa[kHalves];     // scores whose weights come next
  u32x4 pc[kHalves][2];   // weights whose P.V comes next: hi part
  u32x4 pcl[kHalves][2];  // and lo part (split_weights), where carried
  // Chunks 0..2 of a step's second sub-tile are read during its first.
  u32x4 kpre[3], vpre[3];
  auto substep = [&](const WideTile& kst, int kh, const WideTile& vst, int vh, int jw,
                     auto with_scores, auto masked, auto first_half) {
    constexpr bool kScores = decltype(with_scores)::value;
    // first_half: this sub-tile reads its own first chunks and, in its last
    // slots, the next sub-tile's (the other half of the same stages);
    // otherwise they were read by the previous sub-tile.
    constexpr bool kFirst = decltype(first_half)::value;
    // Weights go to P.V as hi + lo pairs (split_weights) in the masked steps.
    // The steady steps round them to the input type: they run only in items
    // whose every row sees at least kRoundedMinKeys keys (below, t_steady),
    // where a weight's rounding (at most 2^-8 of itself in bf16) is spread
    // over many keys, and a second P.V product would cost the steady loop a
    // third more matrix-core work (measured: the 64/8-head chunked prefill
    // over 32K-token contexts 8.04 -> 11.3 ms with it in every step, the
    // multi-turn prefill 0.81 -> 1.04 ms).
    constexpr bool kLo = decltype(masked)::value;
    settle_scores(sa);
    if constexpr (decltype(masked)::value) {
      const int key0 = jw * 32;
      if (key0 + 32 > full_end) mask(key0, sa);
    }
    const char* kl = reinterpret_cast<const char*>(kst) + kh * 32 * kRowBytes;
    const char* vl = reinterpret_cast<const char*>(vst) + vh * 32 * kRowBytes;
    f32x16 sb[kHalves];
    u32x4 kop[8], vop[8];
    // operands of chunk c (K dims 16c.., V keys/dims (c/4, c%4)) of the
    // sub-tile at kb / vb
    auto read_at = [&](const char* kb, const char* vb, int c, u32x4& kd,
                       u32x4& vd) __attribute__((always_inline)) {
      if constexpr (kScores) kd = *reinterpret_cast<const u32x4*>(kb - kKBias + k_rdb[c]);
      const char* vp = vb + v_rd[c & 3] + (c >> 2) * 16 * kRowBytes;
      const u32x2 lo = ds_read_tr(reinterpret_cast<const uint16_t*>(vp));
      const u32x2 hi = ds_read_tr(reinterpret_cast<const uint16_t*>(vp + 4 * kRowBytes));
      vd = u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    auto read = [&](auto C) __attribute__((always_inline)) {
      constexpr int c = decltype(C)::value;
      if constexpr (c < 8)
        read_at(kl, vl, c, kop[c], vop[c]);
      else if constexpr (kFirst)
        read_at(kl + 32 * kRowBytes, vl + 32 * kRowBytes, c - 8, kpre[c - 8], vpre[c - 8]);
    };
    // Weights of `sa`, in slices, against the current reference max.  A row
    // needs a new reference only when its max grew by more than 2^8 in
    // weight, which after a row's first keys is rare.  Such a weight makes
    // its lane's sum of weights exceed 2^7, so the row maxima are found only
    // when some lane's sum does (below): then the wave finds them, moves the
    // references that must move, and redoes its weights (bit for bit the
    // same ones where no reference moved).
    // The row sums add the fp32 weights: a packed dot product would round
    // them like the products' operands, but it issues to the matrix-core pipe
    // and stalls it (about 16 cycles each, measured), while the adds run
    // beside the products.
    float mt[kHalves], sum[kHalves];
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) sum[hh] = 0.f;
    u32x4 pn[kHalves][2], pnl[kHalves][2];
    auto weights = [&](int hh, int e) {  // keys 2e, 2e+1 of the lane's 16
      const float p0 = fast_exp2(__builtin_fmaf(sa[hh][2 * e], c, -mc[hh]));
      const float p1 = fast_exp2(__builtin_fmaf(sa[hh][2 * e + 1], c, -mc[hh]));
      // The sum's first add sits between the second exponential and the
      // pack, so that no result of an exponential is read by the very next
      // instruction (which would cost a wait state).
      sum[hh] = e == 0 ? p0 : sum[hh] + p0;
      if constexpr (kLo) {
        const u32x2 w = split_weights<T>(p0, p1);
        pn[hh][e >> 2][e & 3] = w[0];
        pnl[hh][e >> 2][e & 3] = w[1];
      } else
        pn[hh][e >> 2][e & 3] = Pair<T>::pack(p0, p1);
      sum[hh] += p1;
      // The adds stay in this slot, beside its products (left to itself,
      // the compiler sinks them all past the last slot as one dependent
      // chain with no product to hide behind).
      asm volatile("" : "+v"(sum[hh]));
    };
    auto max_lo = [&](int hh) {
      const f32x16& v = sa[hh];
      mt[hh] = fmaxf(fmaxf(fmaxf(v[0], v[1]), v[2]), fmaxf(fmaxf(v[3], v[4]), v[5]));
      mt[hh] = fmaxf(fmaxf(mt[hh], v[6]), v[7]);
    };
    auto max_hi = [&](int hh) {
      const f32x16& v = sa[hh];
      float m = fmaxf(fmaxf(fmaxf(v[8], v[9]), v[10]), fmaxf(fmaxf(v[11], v[12]), v[13]));
      mt[hh] = max_xor32(fmaxf(fmaxf(mt[hh], m), fmaxf(v[14], v[15])));
    };
    // Slot i (0 .. 8*kHalves-1) issues the S product (16-dim step
    // i/kHalves, row half i%kHalves) into `sb`, the P.V product (8-key x
    // 32-dim chunk i/kHalves, same half), the LDS operand reads of the chunk
    // three chunks ahead (after a chunk's last half), the weights of keys
    // 2(i/kHalves), +1 of that half, and a quarter of one half's row max
    // (slots 1, 3: half 0; 5, 7: half 1).  A scheduling barrier closes each
    // slot, so the products stay spread evenly through the vector work.
    if constexpr (kFirst) {
      read(Stage<0>{});
      read(Stage<1>{});
      read(Stage<2>{});
    } else {
#pragma unroll
      for (int c2 = 0; c2 < 3; ++c2) {
        kop[c2] = kpre[c2];
        vop[c2] = vpre[c2];
      }
    }
    static_for<0, 8 * kHalves>([&](auto I) {
      constexpr int i = decltype(I)::value;
      constexpr int ck = i / kHalves, hk = i % kHalves;
      if constexpr (kScores) {
        if constexpr (ck == 0)
          sb[hk] = MfmaScores<T>::first(kop[0], qreg[hk][0]);
        else
          MfmaScores<T>::next(sb[hk], kop[ck], qreg[hk][ck]);
      }
      o[hk][ck & 3] = MM::mm32(vop[ck], pc[hk][ck >> 2], o[hk][ck & 3]);
      if constexpr (kLo) o[hk][ck & 3] = MM::mm32(vop[ck], pcl[hk][ck >> 2], o[hk][ck & 3]);
      if constexpr (hk == kHalves - 1) read(Stage<ck + 3>{});
      weights(hk, ck);
      __builtin_amdgcn_sched_barrier(0);
    });
    // Keep the weights and sums in the slots above instead of being moved
    // past the branch below.
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        asm volatile("" ::"v"(pn[hh][ks]));
        if constexpr (kLo) asm volatile("" ::"v"(pnl[hh][ks]));
      }
      asm volatile("" ::"v"(sum[hh]));
    }
    float alpha[kHalves];
    bool big = false;
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
      alpha[hh] = 1.f;
      big = big || sum[hh] > 128.f;  // also a non-finite sum
    }
    if (__builtin_amdgcn_ballot_w64(big)) {
      // Some row's max may have grown by more than 2^8: rows that grew move
      // their reference, the weights are redone against it, and O (which now
      // holds P(j) V(j) as well) is taken to the new reference.
#pragma unroll
      for (int hh = 0; hh < kHalves; ++hh) {
        max_lo(hh);
        max_hi(hh);
      }
#pragma unroll
      for (int hh = 0; hh < kHalves; ++hh) {
        const float m_new = (mt[hh] - m_ref[hh]) * c > 8.f ? fmaxf(m_ref[hh], mt[hh]) : m_ref[hh];
        alpha[hh] = fast_exp2((m_ref[hh] - m_new) * c);
        m_ref[hh] = m_new;
        mc[hh] = m_new * c;
        sum[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) weights(hh, e);
      }
      rescale(alpha);
    }
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) {
      l[hh] = l[hh] * alpha[hh] + sum[hh];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pc[hh][ks] = pn[hh][ks];
        if constexpr (kLo) pcl[hh][ks] = pnl[hh][ks];
      }
      if constexpr (kScores) sa[hh] = sb[hh];
    }
  };

  // Prologue: tiles 0..2 in flight, wait for tile 0, weights of sub-tile 0,
  // scores of sub-tile 1.  With 4 waves, waves whose rows all lie past the
  // end compute on mirrored rows and store nothing (only the last workgroup
  // of a (sequence, KV head) has any).
  // (The scheduling barriers keep the loads in this order, which the wait
  // counts below rely on.)
  issue(tab[min(blk, N - 1)], k0, v0);
  __builtin_amdgcn_sched_barrier(0);
  issue(tab[min(4 + blk, N - 1)], k1, v1);
  __builtin_amdgcn_sched_barrier(0);
  int32_t id_next = load_id(3);  // for step 0
  __builtin_amdgcn_sched_barrier(0);
  issue(tab[min(8 + blk, N - 1)], k2, v2);
  __builtin_amdgcn_sched_barrier(0);
  int32_t id_later = load_id(4);  // for step 1
  __builtin_amdgcn_sched_barrier(0);
  // Q is an operand of the products only: it moves to the accumulation
  // registers once its loads (issued first) have landed.
#pragma unroll
  for (int hh = 0; hh < kHalves; ++hh)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) asm volatile("" : "+a"(qreg[hh][kk]));
  wait_vmcnt<2 * (kLoads + 1)>();  // tile 0 (tile 1, id 3, tile 2, id 4 may be in flight)
  pipeline_barrier();
  if (n_tiles == 1) clear_v_tail(v0, 0);
  if (compute) {
    scores(k0, 0, sa);
    settle_scores(sa);
    if (32 > full_end) mask(0, sa);
    float alpha[kHalves];
    softmax(sa, pc, pcl, alpha);  // O is still zero: nothing to rescale
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh) mc[hh] = m_ref[hh] * c;
    scores(k0, 1, sa);
  }
  // Tile step t < n_tiles - 1: sub-tiles j = 2t and 2t+1, which read K of
  // tile t+1 and V of tile t.  Tiles t+2 and t+3 load meanwhile.  The stages
  // are compile-time choices, so every LDS access names one stage array.
  auto step = [&](const int t, WideTile& vcur, WideTile& knxt, WideTile& vnxt, WideTile& kfut,
                  WideTile& vfut, auto masked) {
    wait_vmcnt<kLoads + 1>();  // tile t+1 and the id of tile t+3 landed (tile t+2, id t+4 may not)
    pipeline_barrier();
    issue(id_next, kfut, vfut);  // into the stage of tile t-1, which every wave is done with
    id_next = id_later;
    id_later = load_id(t + 5);
    if (t + 2 == n_tiles) clear_v_tail(vnxt, t + 1);
    if (compute) {
      substep(knxt, 0, vcur, 0, 2 * t + 1, Stage<1>{}, masked, Stage<1>{});
      substep(knxt, 1, vcur, 1, 2 * t + 2, Stage<1>{}, masked, Stage<0>{});
    }
  };
  auto kstage = [&](int i) -> WideTile& {
    return (i & 3) == 0 ? k0 : (i & 3) == 1 ? k1 : (i & 3) == 2 ? k2 : k3;
  };
  auto vstage = [&](int i) -> WideTile& {
    return (i & 3) == 0 ? v0 : (i & 3) == 1 ? v1 : (i & 3) == 2 ? v2 : v3;
  };
  // Steps whose two sub-tiles of weights (keys up to 64t + 95) lie below
  // the keys every row sees need no mask: the steady loop.  The rest, at
  // most the last few of a (sequence, KV head), take the masked step with
  // the stage chosen at run time, where the compiler cannot tell the stages
  // apart and waits for the loads in flight before reading one.  An item
  // whose rows see fewer than kRoundedMinKeys keys takes the masked step
  // throughout, carrying every weight as a hi + lo pair: with few keys an
  // output can be near 1 and rest on a few weights, and one rounded weight
  // could then use up the tolerance by itself.
  const int t_steady =
      full_end < kRoundedMinKeys ? 0 : min(n_tiles - 1, (full_end - 96) / kTileKeys + 1);
  int t = 0;
  for (;; t += 4) {
    if (t >= t_steady) break;
    step(t, v0, k1, v1, k3, v3, Stage<0>{});
    if (t + 1 >= t_steady) {
      t += 1;
      break;
    }
    step(t + 1, v1, k2, v2, k0, v0, Stage<0>{});
    if (t + 2 >= t_steady) {
      t += 2;
      break;
    }
    step(t + 2, v2, k3, v3, k1, v1, Stage<0>{});
    if (t + 3 >= t_steady) {
      t += 3;
      break;
    }
    step(t + 3, v3, k0, v0, k2, v2, Stage<0>{});
  }
  // The steady steps carried no lo part: the weights they left for the
  // first masked P.V have none.
  if (t > 0) {
#pragma unroll
    for (int hh = 0; hh < kHalves; ++hh)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pcl[hh][ks] = u32x4{0u, 0u, 0u, 0u};
  }
  for (; t < n_tiles - 1; ++t)
    step(t, vstage(t), kstage(t + 1), vstage(t + 1), kstage(t + 3), vstage(t + 3), Stage<1>{});
  {
    // t = n_tiles - 1: weights of its second half and the last two P.V.
    // The barrier makes the other waves' clearing of this tile's V tail
    // visible.  The stage is chosen at run time here, where the compiler
    // cannot tell the stages apart and waits for every load in flight before
    // reading it: two loads past the end, once.
    wait_vmcnt<0>();  // every load has landed, also those past the end
    pipeline_barrier();
    WideTile& vlast = vstage(t);
    if (compute) {
      substep(vlast, 0, vlast, 0, 2 * t + 1, Stage<0>{}, Stage<1>{}, Stage<1>{});  // no scores: K unused
      pv(vlast, 1, pc, pcl);
    }
    pipeline_barrier();  // every LDS read done before the stages are reused
  }

  if (!wave_live) return;
  // Normalise and store: lane l holds dims dt*32 + 8*(v/4) + 4*h + v%4.
#pragma unroll
  for (int hh = 0; hh < kHalves; ++hh) {
    const float lt = sum_xor32(l[hh]);
    if (row_ok[hh]) {
      const float inv = 1.f / lt;
      uint16_t* orow = a.out + ((size_t)(q0 + tok[hh]) * a.Hq + g * a.G + hg[hh]) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 pk;
          pk[0] = Pair<T>::pack(o[hh][dt][q4 * 4 + 0] * inv, o[hh][dt][q4 * 4 + 1] * inv);
          pk[1] = Pair<T>::pack(o[hh][dt][q4 * 4 + 2] * inv, o[hh][dt][q4 * 4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + dt * 32 + q4 * 8 + h * 4) = pk;
        }
    }
  }
}

template <typename T, int kHalves>
__global__ __launch_bounds__(512 / kHalves, 1) void prefill_wide_kernel(
    PrefillArgs args, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ order) {
  // (The LDS layout follows the variables' names: the V tiles, read twice as
  // often, get the low 64 KiB.)
  __shared__ __attribute__((aligned(16))) WideTile a_v0, a_v1, a_v2, a_v3, b_k0, b_k1, b_k2, b_k3;
  __shared__ int next;
  PrefillArgs a = args;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.qsl = qsl;
  a.order = order;
  // Persistent, one workgroup per compute unit: the workgroups of XCD x take
  // the items of that XCD's queue in turn.
  const int x = blockIdx.x & 7;
  for (;;) {
    if (threadIdx.x == 0) next = atomicAdd(a.queue + x, 1);
    __syncthreads();
    const int k = __builtin_amdgcn_readfirstlane(next);
    __syncthreads();  // all have read `next` before it is taken again
    if (k >= a.per_xcd) break;
    attend_wide<T, kHalves>(a, k * 8 + x, b_k0, b_k1, b_k2, b_k3, a_v0, a_v1, a_v2, a_v3);
  }
}

// Ranks the sequences by prefill work, (query tiles) x (64-key tiles), most
// first (ties by index): order[rank] = sequence.  Sequences the decode kernel
// takes (n * G <= 8) have no prefill work and come last.  One thread per
// sequence, each counting the keys ahead of its own; batches of more than
// kOrderMaxSeqs sequences keep their order.  Also empties the 8 XCD queues.
__global__ __launch_bounds__(kOrderMaxSeqs) void prefill_order_kernel(
    const int32_t* context_lens, const int32_t* qsl, int32_t num_seqs, int32_t G,
    int32_t* order, int32_t* queue) {
  __shared__ uint32_t key[kOrderMaxSeqs];
  if (threadIdx.x < 8) queue[threadIdx.x] = 0;
  if (num_seqs > kOrderMaxSeqs) {
    for (int s = threadIdx.x; s < num_seqs; s += kOrderMaxSeqs) order[s] = s;
    return;
  }
  const int s = threadIdx.x;
  uint32_t k = 0;
  if (s < num_seqs) {
    k = prefill_work_key(context_lens[s], qsl[s + 1] - qsl[s], G);
    key[s] = k;
  }
  __syncthreads();
  if (s >= num_seqs) return;
  int rank = 0;
  for (int t = 0; t < num_seqs; ++t) {
    const uint32_t kt = key[t];
    rank += (kt > k) | ((kt == k) & (t < s));
  }
  order[rank] = s;
}

}  // namespace

hipError_t launch_prefill(bool is_bf16, const WorkspaceLayout& ws, void* out, const void* q,
                          const void* k_pool, const void* v_pool, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const int32_t* query_start_loc, int32_t num_seqs,
                          int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                          float scale, void* workspace, hipStream_t stream, bool ranked) {
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
  // Calls with long runs of query rows per KV head take the wide kernel (4
  // waves of 64 rows); calls whose longest run is more than one 128-row
  // tile but shorter than that take its 8-wave form (32 rows per wave), so
  // that a run of up to 256 rows reads its K/V once.
  const bool wide = max_rows >= kWideMinRows;
  const bool mid = !wide && max_rows > kWgRows;
  const int64_t wg_rows = wide || mid ? kWideWgRows : kWgRows;
  args.tiles_per_head = (int32_t)((max_rows + wg_rows - 1) / wg_rows);
  args.num_pairs = num_seqs * num_kv_heads;
  if (args.num_pairs <= 0 || args.tiles_per_head <= 0) return hipSuccess;
  args.scale_log2 = scale * kLog2e;
  args.items = nullptr;
  args.count = nullptr;
  args.max_items = 0;
  args.prefix_rec = nullptr;
  char* base = static_cast<char*>(workspace);
  int32_t* order = reinterpret_cast<int32_t*>(base + ws.order);
  args.order = order;
  args.queue = reinterpret_cast<int32_t*>(base + ws.queue);
  // The ranking and the empty queues come from the decode kernel launched
  // just before (`ranked`), or from a launch of their own.
  if (!ranked) {
    hipLaunchKernelGGL(prefill_order_kernel, dim3(1), dim3(kOrderMaxSeqs), 0, stream,
                       context_lens, query_start_loc, num_seqs, args.G, order, args.queue);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int64_t per_xcd = ((int64_t)args.num_pairs + 7) / 8 * args.tiles_per_head;
  args.per_xcd = (int32_t)per_xcd;
  if (wide || mid) {
    // One workgroup per compute unit: 32 per XCD at most.
    const dim3 grid((unsigned)(8 * (per_xcd < kWideWgsPerXcd ? per_xcd : kWideWgsPerXcd)));
    if (mid) {
      if (is_bf16)
        hipLaunchKernelGGL((prefill_wide_kernel<bf16, 1>), grid, dim3(512), 0, stream, args,
                           block_tables, context_lens, query_start_loc, args.order);
      else
        hipLaunchKernelGGL((prefill_wide_kernel<f16, 1>), grid, dim3(512), 0, stream, args,
                           block_tables, context_lens, query_start_loc, args.order);
    } else {
      if (is_bf16)
        hipLaunchKernelGGL((prefill_wide_kernel<bf16, 2>), grid, dim3(256), 0, stream, args,
                           block_tables, context_lens, query_start_loc, args.order);
      else
        hipLaunchKernelGGL((prefill_wide_kernel<f16, 2>), grid, dim3(256), 0, stream, args,
                           block_tables, context_lens, query_start_loc, args.order);
    }
    return hipGetLastError();
  }
  // Two workgroups fit a compute unit: 64 per XCD (32 compute units) at most.
  const dim3 grid((unsigned)(8 * (per_xcd < kPrefillWgsPerXcd ? per_xcd : kPrefillWgsPerXcd)));
  if (is_bf16)
    hipLaunchKernelGGL((prefill_kernel<bf16, false>), grid, dim3(256), 0, stream, args,
                       block_tables, context_lens, query_start_loc, args.order);
  else
    hipLaunchKernelGGL((prefill_kernel<f16, false>), grid, dim3(256), 0, stream, args,
                       block_tables, context_lens, query_start_loc, args.order);
  return hipGetLastError();
}

hipError_t launch_cascade(bool is_bf16, const WorkspaceLayout& ws, const void* q,
                          const void* k_pool, const void* v_pool, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const int32_t* query_start_loc, int32_t num_seqs,
                          int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                          float scale, void* workspace, hipStream_t stream) {
  char* base = static_cast<char*>(workspace);
  PlanArgs plan;
  plan.block_tables = block_tables;
  plan.context_lens = context_lens;
  plan.qsl = query_start_loc;
  plan.starts = reinterpret_cast<int32_t*>(base + ws.starts);
  plan.items = reinterpret_cast<int32_t*>(base + ws.items);
  plan.count = reinterpret_cast<int32_t*>(base + ws.item_count);
  plan.max_blocks = max_blocks_per_seq;
  plan.max_context_len = max_context_len;
  plan.num_seqs = num_seqs;
  plan.G = num_q_heads / num_kv_heads;
  plan.Hkv = num_kv_heads;
  plan.max_items = ws.max_items;
  hipLaunchKernelGGL(cascade_plan_kernel, dim3((unsigned)((num_seqs + 3) / 4)), dim3(256), 0,
                     stream, plan);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  PrefillArgs args;
  args.q = static_cast<const uint16_t*>(q);
  args.k_pool = static_cast<const uint16_t*>(k_pool);
  args.v_pool = static_cast<const uint16_t*>(v_pool);
  args.block_tables = block_tables;
  args.context_lens = context_lens;
  args.qsl = query_start_loc;
  args.out = nullptr;
  args.max_blocks = max_blocks_per_seq;
  args.Hq = num_q_heads;
  args.Hkv = num_kv_heads;
  args.G = num_q_heads / num_kv_heads;
  args.tiles_per_head = 0;
  args.num_pairs = 0;
  args.per_xcd = 0;
  args.order = nullptr;
  args.queue = nullptr;
  args.scale_log2 = scale * kLog2e;
  args.items = plan.items;
  args.count = plan.count;
  args.max_items = ws.max_items;
  args.prefix_rec = reinterpret_cast<float*>(base + ws.prefix);
  // Two workgroups fit a compute unit (LDS and registers): one round of them.
  const dim3 grid((unsigned)(ws.max_items < kCascadeWorkgroups ? ws.max_items
                                                                : kCascadeWorkgroups));
  if (is_bf16)
    hipLaunchKernelGGL((prefill_kernel<bf16, true>), grid, dim3(256), 0, stream, args,
                       block_tables, context_lens, query_start_loc, args.items);
  else
    hipLaunchKernelGGL((prefill_kernel<f16, true>), grid, dim3(256), 0, stream, args,
                       block_tables, context_lens, query_start_loc, args.items);
  return hipGetLastError();
}

}  // namespace pa
