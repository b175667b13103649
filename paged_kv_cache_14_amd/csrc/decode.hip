// Split-K paged decode for gfx950.
//
// Handles every sequence whose new query rows per KV head, n_s * G, number at
// most 8 (a decode token, a few speculative tokens, or a GQA group).  The
// attention equation (SOSP 2023 PagedAttention explainer,
// "PagedAttentionアルゴリズム") is evaluated block by block through the block
// table: the vLLM kernel's per-block scores followed by an aggregation step
// (same page, "実装のポイント") become, here, a partition of each sequence's
// blocks into chunks whose (running max m, sum l, unnormalised output acc)
// are merged by rescaling with 2^(m_p - M) (KV-cache textbook ch.6: the
// FlashAttention-2 statistics m and l, logsumexp L = m + log l).
//
// Work decomposition.  The batch's (sequence, KV head, block) units are cut
// into equal slices, one per wave (64 lanes) of a grid that the chip holds at
// once (see decode_kernel), so every wave reads as many K/V tiles as any
// other and all end together; a (sequence, KV head) pair cut by a slice edge
// is merged from its slices' records by the last of them to end.
// A (block, head) tile is 16 tokens x 128 dims = 4 KiB contiguous; the wave
// reads it as four coalesced 1 KiB loads, lane l holding dims 8*(l%16) ..
// 8*(l%16)+7 of tokens 4*i + l/16 (i = 0..3).  K and V go straight from HBM to
// registers: each tile is read by exactly one wave, the next tile's loads are
// issued before the current one is used, and the 512 KiB register file of a
// compute unit holds far more in-flight tiles than its 160 KiB LDS could.
// Each query row's dot product is the sum over the 16 lanes of a DPP row
// (four DPP adds).  Each of the wave's four lane-rows keeps its own online
// softmax over its quarter of the keys, so no cross-row exchange happens
// inside the loop; the four states are merged with wave shuffles at the end.
// The G query heads of a KV head (and up to 8 rows in all) share every K/V
// load: a (block, head) tile is read once per GQA group.
#include "pa_device.h"
#include "pa_launch.h"
#include "qpage.h"

namespace pa {

namespace {

constexpr int kRec = kRecFloats;
constexpr int kStages = 2;  // register ring depth (2 and 4 measured equal; 2 uses fewer VGPRs)
constexpr int kMfmaMinRows = 4;     // query rows per (sequence, KV head) from which decode uses MFMA
                                    // (measured: MFMA 1.66x at 8 rows, 1.07x at 4; VALU 1.03x at 2)
constexpr int kWindowSums = 64;     // per-window unit counts a wave keeps in LDS (4096 sequences)
// Least slice length for a longest pair of T blocks: ceil(sqrt(T) / 2).
__host__ __device__ inline int min_slice(int T) {
  int r = (int)__builtin_sqrtf((float)T);
  while (r * r > T) --r;
  while ((r + 1) * (r + 1) <= T) ++r;  // r = floor(sqrt(T)), exact
  return (r + 1) / 2;
}

constexpr int kWholeMax = 32;       // pairs of at most this many blocks (and a slice) are never cut
                                    // (measured: cutting them costs the shared-prefix tails 5%)
// Batches whose pairs are all short -- none much longer than a slice and at
// most kSnakeMaxT blocks, in at most kSnakeMaxSeqs sequences -- are dealt as
// whole pairs, longest first, in snake order (see decode_kernel).
constexpr int kSnakeMaxT = 63;
constexpr int kSnakeMaxSeqs = 4096;

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* qsl;
  uint16_t* out;
  float* ws;            // records of cut pairs [waves][2][R][kRec]
  uint32_t* counters;   // [S][Hkv] slices of a cut pair finished; each call leaves them 0
  const int32_t* starts;     // [S][2] first block to decode, prefix chunks; null: no cascade
  const float* prefix_rec;   // [S][Hkv][G][kPrefixChunks][kRec] shared-prefix records
  int32_t* item_count;       // the shared-prefix plan's item count, reset here
  // Calls that may prefill, with at most kRankInDecodeSeqs sequences: the
  // prefill's order of the sequences and its 8 queue heads, written here
  // (null: the ranking kernel writes them).
  int32_t* order;
  int32_t* queue;
  // Quantized pages (qpage.h), the decode over them only: sequence s's first
  // quant_lens[s] keys are pages page_tables[s][0 ..] of qpool.
  const uint8_t* qpool;
  const int32_t* page_tables;
  const int32_t* quant_lens;
  int32_t max_pages;
  int32_t max_blocks;
  int32_t Hq;
  int32_t Hkv;
  int32_t G;
  int32_t S;
  float scale_log2;
};

// A query row's partial softmax state for 8 dims: max M (base-2 logit
// units), sum of weights L, unnormalised output o.
struct RowState {
  float M, L, o[8];
};

// st = row r of (Mr, Lr, Or); r is a run-time value, so select rather than index.
template <int R>
__device__ inline void pick_row(const float (&Mr)[R], const float (&Lr)[R], const float (&Or)[R][8],
                                int r, RowState& st) {
  st.M = Mr[0];
  st.L = Lr[0];
#pragma unroll
  for (int d = 0; d < 8; ++d) st.o[d] = Or[0][d];
#pragma unroll
  for (int i = 1; i < R; ++i) {
    const bool take = r == i;
    st.M = take ? Mr[i] : st.M;
    st.L = take ? Lr[i] : st.L;
#pragma unroll
    for (int d = 0; d < 8; ++d) st.o[d] = take ? Or[i][d] : st.o[d];
  }
}

// Folds n >= 1 (m, l, acc) records into st with the online-softmax rescaling
// 2^(m - M).  load(q, ml, lo, hi) fetches record q's (m, l) and this lane's 8
// accumulator dims; kFoldBatch records are fetched per round trip.
constexpr int kFoldBatch = 8;
// One batch: the first `valid` of the kFoldBatch records count, the rest
// (repeats) weigh 0.
__device__ inline void fold_batch(RowState& st, int valid, const u32x2 (&ml)[kFoldBatch],
                                  const u32x4 (&lo)[kFoldBatch], const u32x4 (&hi)[kFoldBatch]) {
  float mq[kFoldBatch];
  float Mn = st.M;
#pragma unroll
  for (int i = 0; i < kFoldBatch; ++i) {
    mq[i] = i < valid ? __uint_as_float(ml[i][0]) : kNegBig;
    Mn = fmaxf(Mn, mq[i]);
  }
  const float f = fast_exp2(st.M - Mn);
  st.L *= f;
#pragma unroll
  for (int d = 0; d < 8; ++d) st.o[d] *= f;
#pragma unroll
  for (int i = 0; i < kFoldBatch; ++i) {
    const float fi = fast_exp2(mq[i] - Mn);
    st.L += __uint_as_float(ml[i][1]) * fi;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      st.o[d] += __uint_as_float(lo[i][d]) * fi;
      st.o[d + 4] += __uint_as_float(hi[i][d]) * fi;
    }
  }
  st.M = Mn;
}
template <typename Load>
__device__ inline void fold(RowState& st, int n, Load load) {
  for (int q0 = 0; q0 < n; q0 += kFoldBatch) {
    u32x2 ml[kFoldBatch];
    u32x4 lo[kFoldBatch], hi[kFoldBatch];
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) load(min(q0 + i, n - 1), ml[i], lo[i], hi[i]);
    fold_batch(st, n - q0, ml, lo, hi);
  }
}


// ---- Matrix-core partition (v_mfma_f32_16x16x32, fp32 accumulate) ---------
// Lane l = 16q + j: j is a query row (MFMA column; rows >= `rows` are idle),
// q picks a quarter of the operands.  A 32-key step (two blocks) computes
// S^T = K Q^T as two products: in half H, MFMA row i is key
// 8(i/4) + 4H + i%4 of the step, so lane l's accumulators hold exactly keys
// 8q .. 8q+7 of its query row -- the 8 keys the B operand of O^T = V^T P^T
// needs from it: the weights go to the second product without any exchange.
// K goes from HBM straight into the A-operand layout (the key permutation is
// just an address); V rows are staged in the wave's own LDS rows and read
// transposed (ds_read_b64_tr_b16).  The row max and sum are combined over
// the 4 lane quarters with two shuffles; O^T rescales only when a row's max
// grows by more than 2^8 in weight.  The result leaves through LDS in the
// layout of the VALU path: every lane holds every row's (M, L) and dims
// 8(l%16) .. +7.
constexpr int kRowVd = 144;  // elements per staged V row (288 B: transposing reads spread over banks)


template <typename T, int R>
__device__ __forceinline__ void attend_mfma(const DecodeArgs& a, int g, int s, int q0, int n,
                                            int rows, int C, int b0, int b1, float (&Mr)[R],
                                            float (&Lr)[R], float (&Or)[R][8]) {
  using P = Pair<T>;
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[32 * kRowVd];
  __shared__ float2 ml_lds[16];
  const int lane = threadIdx.x, q = lane >> 4, j = lane & 15;
  const size_t blk_stride = (size_t)a.Hkv * kBlockSize * kHeadDim;
  const size_t head_off = (size_t)g * kBlockSize * kHeadDim;

  // Q^T as the B operand: column j = query row j, dims 32m + 8q .. +7.
  u32x4 qb[4];
  int lim_c = -1;  // last key (absolute index) this lane's query row sees
  if (j < rows) {
    const int tok = j / a.G, hg = j - tok * a.G;
    const uint16_t* qrow = a.q + ((size_t)(q0 + tok) * a.Hq + g * a.G + hg) * kHeadDim + 8 * q;
#pragma unroll
    for (int m = 0; m < 4; ++m) qb[m] = load16(qrow + 32 * m);
    lim_c = C - n + tok;
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) qb[m] = u32x4{0u, 0u, 0u, 0u};
  }

  f32x4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegBig, l = 0.f;
  const float c = a.scale_log2;
  // transposing-read bases: lane (q, j) reads key 8q + j/4 (+4), dims 4(j%4) .. +3 (+16t)
  const uint16_t* tr_base = v_lds + (8 * q + (j >> 2)) * kRowVd + 4 * (j & 3);
  const int32_t* table = a.block_tables + (size_t)s * a.max_blocks;

  // Windows of up to 64 blocks: one table entry per lane, read back with
  // v_readlane (no scalar-load latency in the loop).
  for (int wb = b0; wb < b1; wb += 64) {
  const int nblk = min(64, b1 - wb);
  const int my_phys = lane < nblk ? table[wb + lane] : 0;
  // Keys past the window are masked: the ring's re-read tail steps see none.
  const int lim = min(lim_c, (wb + nblk) * kBlockSize - 1);

  // Register stages: K of both halves (4 + 4 operands) and 8 V chunks per step.
  u32x4 kr[2][8], vr[2][8];
  const int kkey = 8 * (j >> 2) + (j & 3);  // half 0's key of MFMA row j; half 1: +4
  auto load_step = [&](int st, int step) {
    const int c0 = min(2 * step, nblk - 1), c1 = min(2 * step + 1, nblk - 1);
    const int ph0 = __builtin_amdgcn_readlane(my_phys, c0);
    const int ph1 = __builtin_amdgcn_readlane(my_phys, c1);
    // K: row kkey (+4) of the step is token kkey % 16 of block kkey / 16.
    const size_t kbase = (size_t)(kkey >= 16 ? ph1 : ph0) * blk_stride + head_off +
                         (kkey & 15) * kHeadDim + 8 * q;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      kr[st][m] = load16_nt(a.k_pool + kbase + 32 * m);
      kr[st][4 + m] = load16_nt(a.k_pool + kbase + 4 * kHeadDim + 32 * m);
    }
    // V: chunk i is key 4i + q of the step, dims 8j .. +7.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 4 * i + q;
      vr[st][i] = load16_nt(a.v_pool + (size_t)(i < 4 ? ph0 : ph1) * blk_stride + head_off +
                            (key & 15) * kHeadDim + 8 * j);
    }
  };

  auto step = [&](int st, int stp) {
    const int key0 = (wb + 2 * stp) * kBlockSize;  // absolute index of the step's key 0
    // Stage V (keys at or past C may hold anything: stored as 0).
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 4 * i + q;
      const u32x4 v = key0 + key < C ? vr[st][i] : u32x4{0u, 0u, 0u, 0u};
      store16(v_lds + key * kRowVd + 8 * j, v);
    }
    // S^T halves.
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      sa = Mfma16<T>::mm(kr[st][m], qb[m], sa);
      sb = Mfma16<T>::mm(kr[st][4 + m], qb[m], sb);
    }
    float x[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      x[v] = key0 + 8 * q + v <= lim ? sa[v] : -__builtin_inff();
      x[4 + v] = key0 + 8 * q + 4 + v <= lim ? sb[v] : -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__builtin_amdgcn_ballot_w64((mx - m_ref) * c > 8.f)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = fast_exp2((m_ref - m_new) * c);
      m_ref = m_new;
      l *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
    }
    const float mc = m_ref * c;
    u32x4 pb, pl;  // the weights as hi + lo pairs of the input type (split_weights)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = fast_exp2(__builtin_fmaf(x[2 * e], c, -mc));
      const float p1 = fast_exp2(__builtin_fmaf(x[2 * e + 1], c, -mc));
      const u32x2 w = split_weights<T>(p0, p1);
      pb[e] = w[0];
      pl[e] = w[1];
      l += p0 + p1;
    }
    // O^T += V^T P^T, dims 16t .. 16t+15 per product, once for the weights'
    // hi part and once for their lo part.  The staged V rows were written by
    // other lanes of this wave: wait for the LDS writes.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x2 lo = ds_read_tr(tr_base + 16 * t);
      const u32x2 hi = ds_read_tr(tr_base + 4 * kRowVd + 16 * t);
      const u32x4 vop = {lo[0], lo[1], hi[0], hi[1]};
      o[t] = Mfma16<T>::mm(vop, pb, o[t]);
      o[t] = Mfma16<T>::mm(vop, pl, o[t]);
    }
  };

  // Two-stage ring (3 and 4 stages measured 12% and 25% slower: more random
  // tile reads in flight cost the DRAM more than they hide).  The last load
  // re-reads the window's last block; the step after it is never taken.
  const int nsteps = (nblk + 1) / 2;
  load_step(0, 0);
  int stp = 0;
  for (; stp + 1 < nsteps; stp += 2) {
    load_step(1, stp + 1);
    step(0, stp);
    load_step(0, stp + 2);
    step(1, stp + 1);
  }
  if (stp < nsteps) step(0, stp);
  }  // window

  // Hand over through LDS: o[t][v] is row j, dim 16t + 4q + v.
  const float lt = [&] {
    float x = l + __shfl_xor(l, 16);
    return x + __shfl_xor(x, 32);
  }();
  float* o_lds = reinterpret_cast<float*>(v_lds);  // 16 rows x 128 dims fp32 = 8 KiB <= 9 KiB
  __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0): the last transposing reads are done
#pragma unroll
  for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(o_lds + j * kHeadDim + 16 * t + 4 * q) = o[t];
  if (q == 0) ml_lds[j] = float2{m_ref * c, lt};
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  const int lc = lane & 15;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(o_lds + r * kHeadDim + 8 * lc);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(o_lds + r * kHeadDim + 8 * lc + 4);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      Or[r][d] = lo[d];
      Or[r][4 + d] = hi[d];
    }
    const float2 ml = ml_lds[r];
    Mr[r] = ml.x;
    Lr[r] = ml.y;
  }
}

// ---- VALU partition: R <= 2 query rows ---------------------------------------
// Lane l holds dims 8*(l%16) .. +7 of tokens 4i + l/16 of each block; each of
// the four lane-rows keeps its own online softmax over its quarter of the
// keys, merged with wave shuffles at the end.  Leaves every lane holding
// every row's (M, L) and dims 8(l%16) .. +7, like attend_mfma.
template <typename T, int R>
__device__ __forceinline__ void attend_valu(const DecodeArgs& a, int g, int s, int q0, int n,
                                            int rows, int C, int b0, int b1, float (&Mr)[R],
                                            float (&Lr)[R], float (&Or)[R][8]) {
  using P = Pair<T>;
  const int lane = threadIdx.x, lr = lane >> 4, lc = lane & 15;
  const size_t blk_stride = (size_t)a.Hkv * kBlockSize * kHeadDim;
  // Query rows r = token * G + head-in-group; row r sees keys 0 .. lim_c[r].
  u32x4 qv[R];
  int lim_c[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rows) {
      const int tok = r / a.G, hg = r - tok * a.G;
      qv[r] = load16(a.q + ((size_t)(q0 + tok) * a.Hq + g * a.G + hg) * kHeadDim + lc * 8);
      lim_c[r] = C - n + tok;  // causal limit
    } else {
      qv[r] = u32x4{0u, 0u, 0u, 0u};
      lim_c[r] = -1;
    }
  }

  float m[R], ls[R], acc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegBig;
    ls[r] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[r][d] = 0.f;
  }

  const size_t lane_off = (size_t)g * kBlockSize * kHeadDim + lr * kHeadDim + lc * 8;
  const int32_t* table = a.block_tables + (size_t)s * a.max_blocks;

  // Windows of up to 64 blocks: one table entry per lane, read back with
  // v_readlane (no scalar-load latency in the loop).
  for (int wb = b0; wb < b1; wb += 64) {
    const int nblk = min(64, b1 - wb);
    const int my_phys = lane < nblk ? table[wb + lane] : 0;
    int lim[R];  // keys past the window are masked: the ring's re-read tail steps see none
#pragma unroll
    for (int r = 0; r < R; ++r) lim[r] = min(lim_c[r], (wb + nblk) * kBlockSize - 1);

    // Ring of kStages register buffers, statically indexed: while block j is
    // consumed the loads of blocks j+1 .. j+kStages-1 are in flight.  The
    // loads are unconditional (the index is clamped to the last block, whose
    // tile is then re-read from L2) so the wait counts stay exact.
    u32x4 kb[kStages][4], vb[kStages][4];
    auto load_block = [&](int st, int jb) {
      const int phys = __builtin_amdgcn_readlane(my_phys, min(jb, nblk - 1));
      const size_t base = (size_t)phys * blk_stride + lane_off;
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // streamed once: nontemporal
        kb[st][i] = load16_nt(a.k_pool + base + i * 4 * kHeadDim);
        vb[st][i] = load16_nt(a.v_pool + base + i * 4 * kHeadDim);
      }
    };

    auto consume = [&](int st, int blk) {
      // Logits of this lane-row's four tokens for every query row (base 2).
      float x[R][4];
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float d = P::dot2(qv[r][0], kb[st][i][0], 0.f);
          d = P::dot2(qv[r][1], kb[st][i][1], d);
          d = P::dot2(qv[r][2], kb[st][i][2], d);
          d = P::dot2(qv[r][3], kb[st][i][3], d);
          d = row16_sum(d);
          const int key = blk * kBlockSize + i * 4 + lr;
          x[r][i] = (key <= lim[r]) ? d * a.scale_log2 : -__builtin_inff();
        }
      }

      // V rows in fp32; slots at or past C may hold anything and become 0.
      const bool tail = (blk + 1) * kBlockSize > C;
      float vf[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = !tail || (blk * kBlockSize + i * 4 + lr < C);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[i][2 * e] = ok ? P::lo(vb[st][i][e]) : 0.f;
          vf[i][2 * e + 1] = ok ? P::hi(vb[st][i][e]) : 0.f;
        }
      }

#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float mx = fmaxf(fmaxf(x[r][0], x[r][1]), fmaxf(x[r][2], x[r][3]));
        const float mn = fmaxf(m[r], mx);
        const float alpha = fast_exp2(m[r] - mn);
        m[r] = mn;
        const float p0 = fast_exp2(x[r][0] - mn), p1 = fast_exp2(x[r][1] - mn);
        const float p2 = fast_exp2(x[r][2] - mn), p3 = fast_exp2(x[r][3] - mn);
        ls[r] = ls[r] * alpha + ((p0 + p1) + (p2 + p3));
#pragma unroll
        for (int d = 0; d < 8; ++d)
          acc[r][d] = acc[r][d] * alpha + p0 * vf[0][d] + p1 * vf[1][d] + p2 * vf[2][d] +
                      p3 * vf[3][d];
      }
    };

#pragma unroll
    for (int st = 0; st < kStages - 1; ++st) load_block(st, st);
    for (int base = 0; base < nblk; base += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        load_block((u + kStages - 1) % kStages, base + u + kStages - 1);
        // Steps past the window consume a re-read tile whose keys are all
        // masked (lim[] stops at the window end): no branch in the ring.
        consume(u, wb + base + u);
      }
    }
  }  // window

  // Merge the four lane-rows (lanes l, l^16, l^32, l^48 hold the same dims):
  // afterwards every lane holds every row's (M, L, o) for its 8 dims.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    Mr[r] = kNegBig;
    Lr[r] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) Or[r][d] = 0.f;
    if (r >= rows) continue;
    float M = fmaxf(m[r], __shfl_xor(m[r], 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = fast_exp2(m[r] - M);
    float L = ls[r] * f;
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      float o = acc[r][d] * f;
      o += __shfl_xor(o, 16);
      o += __shfl_xor(o, 32);
      Or[r][d] = o;
    }
    Mr[r] = M;
    Lr[r] = L;
  }
}

// Calls f(Stage<I>{}) for I = B .. E-1, in order (compile-time indices).
template <int S> struct Idx { static constexpr int value = S; };
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Idx<B>{});
    static_for<B + 1, E>(f);
  }
}

// ---- Quantized pages (qpage.h) on the matrix cores (v_mfma_f32_16x16x32_f16)
// Blocks [b0, b1) of sequence s lie in its quantized pages; every query row
// sees all of them (the pages hold cached keys only).  A key is
// mn_c + code * step_c per channel, a value mn_t + code * step_t per token:
//   q.k = sum_c q_c mn_c + sum_c (q_c step_c) code_c  (+ 4 (q_c step_c) hi_c
//         on the promoted channels),
//   sum_t p_t v_t = sum_t p_t mn_t + sum_t (p_t step_t) code_t.
// The codes go to the products exactly, as f16 (two per register: one
// and-or into 1024.0 and one packed subtraction, code_operand).  The factors
// q_c step_c and p_t step_t are float32, and go in as f16 hi + lo parts,
// so each factor carries about 22 bits and every product is exact in the
// fp32 accumulation.  Lane l = 16q + j: j is a query row (MFMA column; rows
// >= `rows` are idle), q picks a quarter of the operands.  As in
// attend_mfma, MFMA row i of half H of a 32-key step is key
// 8(i/4) + 4H + i%4 of the step, so lane l's accumulators hold keys
// 8q .. 8q+7 of its row, the B operand of the value product.  The first
// sum, per row and page, and the last, per row, are vector work.  The
// result leaves through LDS in the layout of the VALU path, as attend_mfma's.
// Assumes |q_c step_c| and |p_t step_t| below the f16 range (65504).
template <typename T>
__device__ inline float q_value(uint16_t bits);
template <>
__device__ inline float q_value<f16>(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}
template <>
__device__ inline float q_value<bf16>(uint16_t bits) {
  return __uint_as_float((uint32_t)bits << 16);
}

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

// Codes at bit pairs 0 .. 3 of a page word (bits 2p and 16 + 2p; a word's
// pairs 4 .. 7 come here shifted right by 8) as an A operand of four f16
// pairs.  Pair p is or-ed into the mantissa of 1024.0 where it lies, which
// gives 1024 + code * 4^p exactly, and 1024 is taken off by a packed
// subtraction: the operand holds code * 4^p, and the other operand of the
// product carries the factor 4^-p (exact, a power of two).  masks[p] =
// 0x00030003 << 2p, magic = 0x64006400 (1024.0 twice), both in registers.
__device__ inline u32x4 code_operand(uint32_t w, const uint32_t (&masks)[4], uint32_t magic) {
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t x;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(x) : "v"(w), "v"(masks[p]), "v"(magic));
    const h16x2 h = __builtin_bit_cast(h16x2, x) - h16x2{(_Float16)1024.f, (_Float16)1024.f};
    r[p] = __builtin_bit_cast(uint32_t, h);
  }
  return r;
}

// 4^-p for element e of an operand (pair p = e / 2).
__device__ inline float pair_factor(int e) { return e < 2 ? 1.f : e < 4 ? 0.25f : e < 6 ? 0.0625f : 0.015625f; }

// {hi, lo} f16 pairs of two float32 values: hi = f16(x), lo = f16(x - hi).
__device__ inline u32x2 split_f16(float x0, float x1) {
  const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
  const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
  return u32x2{__builtin_bit_cast(uint32_t, h16x2{h0, h1}),
               __builtin_bit_cast(uint32_t, h16x2{l0, l1})};
}

__device__ inline f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <typename T, int R>
__device__ __forceinline__ void attend_quant(const DecodeArgs& a, int g, int s, int q0, int rows,
                                             int b0, int b1, float (&Mr)[R], float (&Lr)[R],
                                             float (&Or)[R][8]) {
  using P = Pair<T>;
  __shared__ __attribute__((aligned(16))) float o_lds[16 * kHeadDim];
  __shared__ float2 qml_lds[16];
  const int lane = threadIdx.x, q = lane >> 4, j = lane & 15;
  // The code operands' constants, kept in registers (code_operand).
  uint32_t masks[4], magic;
#pragma unroll
  for (int p = 0; p < 4; ++p) masks[p] = __builtin_amdgcn_readfirstlane(0x00030003u << (2 * p));
  magic = __builtin_amdgcn_readfirstlane(0x64006400u);
  // Query row j at the lane's channels 32m + 8q + e, as pairs of the input
  // type (idle rows: zero).
  u32x4 qv[4];
  const uint16_t* qrow = nullptr;
  if (j < rows) {
    const int tok = j / a.G, hg = j - tok * a.G;
    qrow = a.q + ((size_t)(q0 + tok) * a.Hq + g * a.G + hg) * kHeadDim;
#pragma unroll
    for (int m = 0; m < 4; ++m) qv[m] = load16(qrow + 32 * m + 8 * q);
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) qv[m] = u32x4{0u, 0u, 0u, 0u};
  }
  f32x4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegBig, l = 0.f, accmn = 0.f;
  const float c = a.scale_log2;
  const int32_t* ptab = a.page_tables + (size_t)s * a.max_pages;
  const int key_lo = b0 * kBlockSize, key_hi = b1 * kBlockSize;

  // Per page: B operands q_c step_c (hi, lo) of the lane's channels, the
  // promoted slots' 4 q_c step_c, and the row's bias sum_c q_c mn_c.
  u32x4 qsh[4], qsl[4], bqh = {0u, 0u, 0u, 0u}, bql = {0u, 0u, 0u, 0u};
  float bias = 0.f;
  auto load_page = [&](const uint8_t* qp) {
    float part = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float qf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[2 * e] = P::lo(qv[m][e]);
        qf[2 * e + 1] = P::hi(qv[m][e]);
      }
      const f32x4 st0 = *reinterpret_cast<const f32x4*>(qp + kQKScale + 4 * (32 * m + 8 * q));
      const f32x4 st1 = *reinterpret_cast<const f32x4*>(qp + kQKScale + 4 * (32 * m + 8 * q + 4));
      const f32x4 mn0 = *reinterpret_cast<const f32x4*>(qp + kQKMin + 4 * (32 * m + 8 * q));
      const f32x4 mn1 = *reinterpret_cast<const f32x4*>(qp + kQKMin + 4 * (32 * m + 8 * q + 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = __builtin_fmaf(qf[e], mn0[e], part);
        part = __builtin_fmaf(qf[4 + e], mn1[e], part);
      }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        // channel 32m + 8q + e sits in pair e / 2 of its code operand
        const float f0 = pair_factor(2 * pp), f1 = pair_factor(4 + 2 * pp);
        const u32x2 w0 =
            split_f16(qf[2 * pp] * st0[2 * pp] * f0, qf[2 * pp + 1] * st0[2 * pp + 1] * f0);
        const u32x2 w1 =
            split_f16(qf[4 + 2 * pp] * st1[2 * pp] * f1, qf[5 + 2 * pp] * st1[2 * pp + 1] * f1);
        qsh[m][pp] = w0[0];
        qsl[m][pp] = w0[1];
        qsh[m][2 + pp] = w1[0];
        qsl[m][2 + pp] = w1[1];
      }
    }
    part += __shfl_xor(part, 16);
    bias = part + __shfl_xor(part, 32);
    // Promoted slots 8q .. 8q+7 (lanes q < 2): 4 q_c step_c at channel boost[slot].
    if (q < 2 && qrow) {
      float bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ch = qp[kQBoostList + 8 * q + e];
        bv[e] = 4.f * pair_factor(e) * q_value<T>(qrow[ch]) *
                *reinterpret_cast<const float*>(qp + kQKScale + 4 * ch);
      }
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const u32x2 w = split_f16(bv[2 * pp], bv[2 * pp + 1]);
        bqh[pp] = w[0];
        bql[pp] = w[1];
      }
    }
  };

  // A step's codes and value parameters, loaded one step ahead.
  struct StepData {
    u32x4 kw, vw;
    uint32_t hw;
    f32x4 vs0, vs1, vm0, vm1;
  };
  auto load_step = [&](const uint8_t* qp, int sp) {
    StepData d;
    d.kw = *reinterpret_cast<const u32x4*>(qp + kQKLo + sp * 1024 + lane * 16);
    d.hw = q < 2 ? *reinterpret_cast<const uint32_t*>(qp + kQKHi + sp * 128 + lane * 4) : 0u;
    d.vw = *reinterpret_cast<const u32x4*>(qp + kQVLo + sp * 1024 + lane * 16);
    d.vs0 = *reinterpret_cast<const f32x4*>(qp + kQVScale + 4 * (32 * sp + 8 * q));
    d.vs1 = *reinterpret_cast<const f32x4*>(qp + kQVScale + 4 * (32 * sp + 8 * q + 4));
    d.vm0 = *reinterpret_cast<const f32x4*>(qp + kQVMin + 4 * (32 * sp + 8 * q));
    d.vm1 = *reinterpret_cast<const f32x4*>(qp + kQVMin + 4 * (32 * sp + 8 * q + 4));
    return d;
  };

  auto step = [&](int st, const StepData& d) {
    // S^T halves: keys 8q + v (sa) and 8q + 4 + v (sb) of row j.
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t w0 = d.kw[m >> 1], w1 = d.kw[2 + (m >> 1)];
      const u32x4 a0 = code_operand((m & 1) ? w0 >> 8 : w0, masks, magic);
      const u32x4 a1 = code_operand((m & 1) ? w1 >> 8 : w1, masks, magic);
      sa = mfma_f16(a0, qsh[m], sa);
      sa = mfma_f16(a0, qsl[m], sa);
      sb = mfma_f16(a1, qsh[m], sb);
      sb = mfma_f16(a1, qsl[m], sb);
    }
    {
      const u32x4 h0 = code_operand(d.hw, masks, magic), h1 = code_operand(d.hw >> 8, masks, magic);
      sa = mfma_f16(h0, bqh, sa);
      sa = mfma_f16(h0, bql, sa);
      sb = mfma_f16(h1, bqh, sb);
      sb = mfma_f16(h1, bql, sb);
    }
    const int key0 = 32 * st + 8 * q;
    float x[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      x[v] = sa[v] + bias;
      x[4 + v] = sb[v] + bias;
    }
    // Only the range's first and last steps hold keys outside it (a branch,
    // kept one by the empty asm: the compiler would rather predicate it).
    if (32 * st < key_lo || 32 * st + 32 > key_hi) {
      asm volatile("");
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        x[v] = key0 + v >= key_lo && key0 + v < key_hi ? x[v] : -__builtin_inff();
        x[4 + v] = key0 + 4 + v >= key_lo && key0 + 4 + v < key_hi ? x[4 + v] : -__builtin_inff();
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__builtin_amdgcn_ballot_w64((mx - m_ref) * c > 8.f)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = fast_exp2((m_ref - m_new) * c);
      m_ref = m_new;
      l *= alpha;
      accmn *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
    }
    const float mc = m_ref * c;
    float pk[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) pk[v] = fast_exp2(__builtin_fmaf(x[v], c, -mc));
    u32x4 pbh, pbl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // key 8q + 2e (+1) sits in pair e of the value code operands
      const float f = pair_factor(2 * e);
      const float w0 = pk[2 * e] * (e < 2 ? d.vs0[2 * e] : d.vs1[2 * e - 4]) * f;
      const float w1 = pk[2 * e + 1] * (e < 2 ? d.vs0[2 * e + 1] : d.vs1[2 * e - 3]) * f;
      const u32x2 w = split_f16(w0, w1);
      pbh[e] = w[0];
      pbl[e] = w[1];
    }
    l += ((pk[0] + pk[1]) + (pk[2] + pk[3])) + ((pk[4] + pk[5]) + (pk[6] + pk[7]));
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      accmn = __builtin_fmaf(pk[v], d.vm0[v], accmn);
      accmn = __builtin_fmaf(pk[4 + v], d.vm1[v], accmn);
    }
    // O^T += Vc^T (p step)^T, dims 16t .. 16t+15 per product.
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t vwt = d.vw[t >> 1];
      const u32x4 av = code_operand((t & 1) ? vwt >> 8 : vwt, masks, magic);
      o[t] = mfma_f16(av, pbh, o[t]);
      o[t] = mfma_f16(av, pbl, o[t]);
    }
  };

  // Windows of up to 64 pages: one page-table entry per lane, read back with
  // v_readlane.  Steps of 32 keys (4 per page); the next step's loads are in
  // flight while one is consumed (the last is loaded again, in vain).
  const int st_first = key_lo / 32, st_end = (key_hi + 31) / 32;
  for (int wst = st_first; wst < st_end; wst += 4 * 64 - (wst & 3)) {
    const int wpg = wst / 4;
    const int wst_end = min(st_end, 4 * (wpg + 64));
    const int my_page = lane < (wst_end + 3) / 4 - wpg ? ptab[wpg + lane] : 0;
    auto page_ptr = [&](int st) {
      const int pg = __builtin_amdgcn_readlane(my_page, st / 4 - wpg);
      return a.qpool + ((size_t)pg * a.Hkv + g) * kQPageBytes;
    };
    StepData cur = load_step(page_ptr(wst), wst & 3);
    load_page(page_ptr(wst));
    for (int st = wst; st < wst_end; ++st) {
      const int sn = min(st + 1, wst_end - 1);
      const StepData nxt = load_step(page_ptr(sn), sn & 3);
      if (st != wst && (st & 3) == 0) load_page(page_ptr(st));
      step(st, cur);
      cur = nxt;
    }
  }

  // Hand over through LDS: o[t][v] is row j, dim 16t + 4q + v; sum_t p_t mn_t
  // joins every dim.
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  float mt = accmn + __shfl_xor(accmn, 16);
  mt += __shfl_xor(mt, 32);
#pragma unroll
  for (int t = 0; t < 8; ++t)
    *reinterpret_cast<f32x4*>(o_lds + j * kHeadDim + 16 * t + 4 * q) =
        o[t] + f32x4{mt, mt, mt, mt};
  if (q == 0) qml_lds[j] = float2{m_ref * c, lt};
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  const int lc = lane & 15;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(o_lds + r * kHeadDim + 8 * lc);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(o_lds + r * kHeadDim + 8 * lc + 4);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      Or[r][d] = lo[d];
      Or[r][4 + d] = hi[d];
    }
    const float2 ml = qml_lds[r];
    Mr[r] = ml.x;
    Lr[r] = ml.y;
  }
  // The next use of o_lds (another range of this wave) writes it only after
  // these reads: a wave's LDS accesses complete in order.
}

// (M1, L1, O1) <- the merge of itself with (M2, L2, O2), row by row.
template <int R>
__device__ inline void merge_rows(float (&M1)[R], float (&L1)[R], float (&O1)[R][8],
                                  const float (&M2)[R], const float (&L2)[R],
                                  const float (&O2)[R][8]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float M = fmaxf(M1[r], M2[r]);
    const float f1 = fast_exp2(M1[r] - M), f2 = fast_exp2(M2[r] - M);
    L1[r] = L1[r] * f1 + L2[r] * f2;
#pragma unroll
    for (int d = 0; d < 8; ++d) O1[r][d] = O1[r][d] * f1 + O2[r][d] * f2;
    M1[r] = M;
  }
}

// Blocks [b0, b1) of sequence s: those in quantized pages through
// attend_quant, the rest (16-bit) through the VALU or matrix-core path.
template <typename T, int R, bool kMfma, bool kQuant>
__device__ __forceinline__ void attend_range(const DecodeArgs& a, int g, int s, int q0, int n,
                                             int rows, int C, int b0, int b1, float (&Mr)[R],
                                             float (&Lr)[R], float (&Or)[R][8]) {
  auto plain = [&](int c0, int c1, float (&M)[R], float (&L)[R], float (&O)[R][8]) {
    if constexpr (kMfma)
      attend_mfma<T, R>(a, g, s, q0, n, rows, C, c0, c1, M, L, O);
    else
      attend_valu<T, R>(a, g, s, q0, n, rows, C, c0, c1, M, L, O);
  };
  if constexpr (kQuant) {
    const int qb = a.quant_lens[s] / kBlockSize;  // blocks held by quantized pages
    if (b0 < qb) {
      attend_quant<T, R>(a, g, s, q0, rows, b0, min(b1, qb), Mr, Lr, Or);
      if (b1 > qb) {
        // The quantized part's state waits in LDS while the 16-bit part
        // runs (held in registers it would push the matrix-core path into
        // spilling); then the two merge.
        __shared__ float park[R * 10][64];
        const int lane = threadIdx.x;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          park[r * 10][lane] = Mr[r];
          park[r * 10 + 1][lane] = Lr[r];
#pragma unroll
          for (int d = 0; d < 8; ++d) park[r * 10 + 2 + d][lane] = Or[r][d];
        }
        plain(qb, b1, Mr, Lr, Or);
        float M1[R], L1[R], O1[R][8];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          M1[r] = park[r * 10][lane];
          L1[r] = park[r * 10 + 1][lane];
#pragma unroll
          for (int d = 0; d < 8; ++d) O1[r][d] = park[r * 10 + 2 + d][lane];
        }
        merge_rows<R>(Mr, Lr, Or, M1, L1, O1);
      }
      return;
    }
  }
  plain(b0, b1, Mr, Lr, Or);
}

// ---- Work split: equal slices of the batch's (KV head, block) stream ---------
// Decode work is the stream of (sequence s, KV head g, block b) units in
// that order, Hkv * T_s units per sequence, where T_s is the number of blocks
// it decodes (the blocks after its shared prefix, if any; 0 for sequences
// the prefill kernel takes).  Wave w of the grid takes units
// [w*chunk, (w+1)*chunk): every wave reads the same number of K/V tiles, so
// all waves of the grid, which is sized to be resident at once, end
// together.  The slice runs over one or more (sequence, KV head) pairs:
// a pair wholly inside it is finished in place, a pair cut by a slice edge
// leaves one (m, l, acc) record per slice, merged by whichever of its
// waves ends last.

// One 64-sequence window of the batch in LDS, one sequence per column.
enum WinField { kWinT, kWinC, kWinQ0, kWinN, kWinStart, kWinChunks, kWinExcl, kWinFields };
using SeqWindow = int[kWinFields][64];
//   kWinT       blocks the sequence decodes per KV head (0: none)
//   kWinExcl    units of the window's sequences before this one

// Blocks sequence s decodes per KV head, from its query rows n, context C
// and first block left to decode.
__device__ inline int decode_blocks(const DecodeArgs& a, int n, int C, int start) {
  const int rows = n * a.G;
  // never past the table row, whatever C says
  const int N = min((C + kBlockSize - 1) / kBlockSize, a.max_blocks);
  // larger runs of rows belong to the prefill kernel
  return rows > 0 && rows <= kDecodeRows && N > start ? N - start : 0;
}

__device__ inline uint32_t wave_sum(uint32_t x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x += __shfl_xor(x, d);
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}

__device__ inline int wave_max(int x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x = max(x, __shfl_xor(x, d));
  return __builtin_amdgcn_readfirstlane(x);
}

// Fills win with sequences first .. first+63; returns the window's units.
__device__ inline uint32_t load_window(const DecodeArgs& a, int first, SeqWindow& win) {
  const int lane = threadIdx.x, s = first + lane;
  int T = 0, C = 0, q0 = 0, n = 0, start = 0, chunks = 0;
  if (s < a.S) {
    q0 = a.qsl[s];
    const int q1 = a.qsl[s + 1];
    C = a.context_lens[s];
    if (a.starts) {
      start = a.starts[2 * s];
      chunks = a.starts[2 * s + 1];
    }
    n = q1 - q0;
    T = decode_blocks(a, n, C, start);
  }
  // inclusive scan of the units over the lanes
  const uint32_t u = (uint32_t)T * (uint32_t)a.Hkv;
  uint32_t x = u;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  win[kWinT][lane] = T;
  win[kWinC][lane] = C;
  win[kWinQ0][lane] = q0;
  win[kWinN][lane] = n;
  win[kWinStart][lane] = start;
  win[kWinChunks][lane] = chunks;
  win[kWinExcl][lane] = (int)(x - u);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Wave-uniform field f of the window's sequence L (one LDS broadcast).
__device__ inline int win_at(const SeqWindow& win, int f, int L) {
  return __builtin_amdgcn_readfirstlane(win[f][L]);
}

// Decode over an equal slice of the unit stream per wave.  kMfma false: the
// VALU partition (attend_valu).  kMfma true: the matrix-core partition
// (attend_mfma), for GQA groups and speculative rows, where the VALU path
// spends about 130 instructions per key on 4 rows.
template <typename T, int R, bool kMfma, bool kQuant>
// Occupancy the planner's grid counts on: two waves per SIMD for 1-2 rows,
// one for the matrix-core instances (measured best; they may then use up to
// 512 registers and take about 300 without spilling).  kQuant: sequences
// begin with quantized pages (attend_range).
__global__ __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(R <= 2 ? 2 : 1))) void decode_kernel(DecodeArgs a) {
  using P = Pair<T>;
  const int lane = threadIdx.x, lr = lane >> 4, lc = lane & 15;
  const int w = blockIdx.x, nw = gridDim.x;
  // The shared-prefix pass has read its plan: clear the count for the next call.
  if (a.item_count && w == 0 && lane == 0) *a.item_count = 0;
  // The prefill launched after this kernel takes its sequences by decreasing
  // work (prefill_work_key), from empty queues: lane l ranks sequence l.
  if (a.order && w == nw - 1) {
    if (lane < 8) a.queue[lane] = 0;
    const uint32_t k =
        lane < a.S ? prefill_work_key(a.context_lens[lane], a.qsl[lane + 1] - a.qsl[lane], a.G)
                   : 0u;
    int rank = 0;
    for (int t = 0; t < a.S; ++t) {
      const uint32_t kt = (uint32_t)__builtin_amdgcn_readlane((int)k, t);
      rank += (kt > k) | ((kt == k) & (t < lane));
    }
    if (lane < a.S) a.order[rank] = lane;
  }

  // Units of every window (the first kWindowSums kept in LDS) and in all.
  __shared__ uint32_t win_units[kWindowSums];
  __shared__ SeqWindow win;
  // Blocks each sequence decodes per KV head (up to kSnakeMaxSeqs sequences,
  // saturated at 255) and, for snake order, how many sequences decode t.
  __shared__ uint8_t t_lds[kSnakeMaxSeqs];
  __shared__ uint32_t t_cnt[64];
  const int nwin = (a.S + 63) / 64;
  uint32_t total = 0;
  int max_t = 0;  // the longest pair's blocks
  // One window: load it whole.  More: four per round trip, only their unit
  // counts kept, then the one holding the slice's start.
  if (nwin == 1) {
    total = load_window(a, 0, win);
    if (lane == 0) win_units[0] = total;
    max_t = wave_max(win[kWinT][lane]);
    if (lane < a.S) t_lds[lane] = (uint8_t)min(win[kWinT][lane], 255);
  }
  for (int r0 = 0; nwin > 1 && r0 < nwin; r0 += 4) {
    // Every load of the four windows first (indices clamped to the last
    // sequence), so that they take one round trip rather than one each.
    int q0[4], q1[4], cl[4], st[4], nb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int sc = min(64 * (r0 + k) + lane, a.S - 1);
      q0[k] = a.qsl[sc];
      q1[k] = a.qsl[sc + 1];
      cl[k] = a.context_lens[sc];
      st[k] = a.starts ? a.starts[2 * sc] : 0;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = 64 * (r0 + k) + lane;
      nb[k] = s < a.S ? decode_blocks(a, q1[k] - q0[k], cl[k], st[k]) : 0;
      if (s < a.S && s < kSnakeMaxSeqs) t_lds[s] = (uint8_t)min(nb[k], 255);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t t = wave_sum((uint32_t)nb[k] * (uint32_t)a.Hkv);
      if (lane == 0 && r0 + k < kWindowSums) win_units[r0 + k] = t;
      total += t;
      max_t = max(max_t, wave_max(nb[k]));
    }
  }
  // Equal slices, but none shorter than about sqrt(T)/2 blocks for the
  // longest pair's T (waves past the end then have nothing to do): the last
  // of a pair's slices folds all their records, so a pair cut into n slices
  // costs ~n/8 dependent round trips after ~T/n blocks of streaming per
  // wave, and n ~ 2 sqrt(T) balances the two.
  const uint32_t chunk = max(max((uint32_t)kMinChunk, (total + nw - 1) / (uint32_t)nw),
                             (uint32_t)min_slice(max_t));
  // A (sequence, KV head) pair and what finishing its rows needs.
  struct PairRef {
    int s, g, q0, n, chunks, Tl;
    uint32_t p0;  // the pair's first unit
  };
  auto write_out = [&](const PairRef& pr, int row, const RowState& st) {
    const int tok = row / a.G, hg = row - tok * a.G;
    const float inv = 1.f / st.L;
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = P::pack(st.o[2 * e] * inv, st.o[2 * e + 1] * inv);
    store16(a.out + ((size_t)(pr.q0 + tok) * a.Hq + pr.g * a.G + hg) * kHeadDim + lc * 8, pk);
  };
  // Shared-prefix records were written by an earlier kernel: plain loads see them.
  auto fold_prefix = [&](const PairRef& pr, int row, RowState& st) {
    // one query token: the row is the head in the group
    const float* pre =
        a.prefix_rec + (((size_t)pr.s * a.Hkv + pr.g) * a.G + row) * kPrefixChunks * kRec;
    fold(st, pr.chunks, [&](int cq, u32x2& ml, u32x4& lo, u32x4& hi) {
      const float* rc = pre + cq * kRec;
      ml = *reinterpret_cast<const u32x2*>(rc + 128);
      lo = load16(rc + lc * 8);
      hi = load16(rc + lc * 8 + 4);
    });
  };

  // Short pairs only: whole pairs, dealt longest first in snake order.  Pair
  // ranks order sequences by decreasing blocks (ties by index) and a
  // sequence's pairs by KV head; wave w takes ranks w, 2nw-1-w, 2nw+w, ...,
  // so a long pair of one round goes with a short one of the next, and no
  // pair is cut (no records, no tickets).  With equal slices a wave owns the
  // pairs that start in its slice, which here leaves the busiest wave near
  // twice the mean work.
  // (Equal slices leave the busiest wave up to about chunk + min(chunk, 32)
  // units; snake order leaves it the longest pair.)
  if (max_t <= (int)chunk + min((int)chunk, kWholeMax) / 2 && max_t <= kSnakeMaxT &&
      a.S <= kSnakeMaxSeqs) {
    t_cnt[lane] = 0;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): one wave, its own LDS writes
    __builtin_amdgcn_wave_barrier();
    for (int s = lane; s < a.S; s += 64) {
      const int t = t_lds[s];
      if (t > 0) atomicAdd(&t_cnt[t], 1u);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    // ge (lane t >= 1): sequences that decode at least t blocks
    uint32_t ge = t_cnt[lane];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_down(ge, d);
      if (lane + d < 64) ge += y;
    }
    const uint32_t n_pairs = (uint32_t)__builtin_amdgcn_readlane((int)ge, 1) * (uint32_t)a.Hkv;
    for (uint32_t k = 0;; ++k) {
      const uint32_t base = k * (uint32_t)nw;
      if (base >= n_pairs) break;
      const uint32_t p = base + ((k & 1) ? (uint32_t)(nw - 1 - w) : (uint32_t)w);
      if (p >= n_pairs) continue;
      const uint32_t rank = p / (uint32_t)a.Hkv;
      const int g = (int)(p - rank * (uint32_t)a.Hkv);
      // The sequence of rank `rank`: its block count t is the largest with
      // ge[t] > rank, and it is the kk-th of those with t blocks.
      const uint64_t above = __builtin_amdgcn_ballot_w64(lane >= 1 && ge > rank);
      const int t = 63 - __builtin_clzll(above);
      uint32_t kk = rank - (t < 63 ? (uint32_t)__builtin_amdgcn_readlane((int)ge, t + 1) : 0u);
      int sq = -1;
      for (int s0 = 0; s0 < a.S; s0 += 64) {
        const int i = s0 + lane;
        const uint64_t m = __builtin_amdgcn_ballot_w64(i < a.S && t_lds[i] == t);
        const uint32_t c = (uint32_t)__builtin_popcountll(m);
        if (kk < c) {
          const uint32_t below =
              __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          const uint64_t hit = __builtin_amdgcn_ballot_w64(((m >> lane) & 1) && below == kk);
          sq = s0 + __builtin_ctzll(hit);
          break;
        }
        kk -= c;
      }
      if (sq < 0) break;  // unreachable: the counts came from t_lds
      PairRef pr;
      pr.s = __builtin_amdgcn_readfirstlane(sq);
      pr.g = __builtin_amdgcn_readfirstlane(g);
      pr.q0 = a.qsl[pr.s];
      pr.n = a.qsl[pr.s + 1] - pr.q0;
      pr.chunks = a.starts ? a.starts[2 * pr.s + 1] : 0;
      pr.Tl = t;
      pr.p0 = 0;
      const int C = a.context_lens[pr.s];
      const int b0 = a.starts ? a.starts[2 * pr.s] : 0;  // b0 + t: the sequence's last block
      const int rows = pr.n * a.G;
      // The first two prefix records the rows fold in at the end were written
      // by an earlier kernel: their loads go out with the pair's first K/V
      // loads instead of after them.
      constexpr int kRowsPerLane = (R + 3) / 4;
      struct PreRec {
        u32x2 ml0, ml1;
        u32x4 lo0, lo1, hi0, hi1;
      };
      PreRec pre[kRowsPerLane];
      if (!kQuant && pr.chunks > 0) {  // quantized-page calls hold no groups
#pragma unroll
        for (int kr = 0; kr < kRowsPerLane; ++kr) {
          const int row = min(lr + 4 * kr, rows - 1);
          const float* rec =
              a.prefix_rec + (((size_t)pr.s * a.Hkv + pr.g) * a.G + row) * kPrefixChunks * kRec;
          const float* r1 = rec + min(1, pr.chunks - 1) * kRec;
          pre[kr].ml0 = *reinterpret_cast<const u32x2*>(rec + 128);
          pre[kr].lo0 = load16(rec + lc * 8);
          pre[kr].hi0 = load16(rec + lc * 8 + 4);
          pre[kr].ml1 = *reinterpret_cast<const u32x2*>(r1 + 128);
          pre[kr].lo1 = load16(r1 + lc * 8);
          pre[kr].hi1 = load16(r1 + lc * 8 + 4);
        }
      }
      float Mr[R], Lr[R], Or[R][8];
      attend_range<T, R, kMfma, kQuant>(a, pr.g, pr.s, pr.q0, pr.n, rows, C, b0, b0 + t, Mr,
                                        Lr, Or);
#pragma unroll
      for (int kr = 0; kr < kRowsPerLane; ++kr) {
        const int row = lr + 4 * kr;
        if (row >= rows) continue;
        RowState st;
        pick_row<R>(Mr, Lr, Or, row, st);
        if (kQuant || pr.chunks > 2) {
          if (pr.chunks > 0) fold_prefix(pr, row, st);
        } else if (pr.chunks > 0) {  // the loaded-ahead records, the rest repeats
          u32x2 ml[kFoldBatch];
          u32x4 lo[kFoldBatch], hi[kFoldBatch];
          ml[0] = pre[kr].ml0;
          lo[0] = pre[kr].lo0;
          hi[0] = pre[kr].hi0;
#pragma unroll
          for (int i = 1; i < kFoldBatch; ++i) {
            ml[i] = pre[kr].ml1;
            lo[i] = pre[kr].lo1;
            hi[i] = pre[kr].hi1;
          }
          fold_batch(st, pr.chunks, ml, lo, hi);
        }
        write_out(pr, row, st);
      }
    }
    return;
  }

  const uint32_t u0 = (uint32_t)w * chunk;
  if (u0 >= total) return;
  const uint32_t u1 = min(u0 + chunk, total);

  // The window holding unit u0 and its first unit.
  int r = 0;
  uint32_t wbase = 0, wtot = 0;
  for (;; ++r) {
    wtot = r < kWindowSums ? win_units[r] : load_window(a, 64 * r, win);
    wtot = __builtin_amdgcn_readfirstlane(wtot);
    if (wbase + wtot > u0 || r + 1 == nwin) break;
    wbase += wtot;
  }
  if (nwin > 1) load_window(a, 64 * r, win);
  // its sequence: the one whose units contain u0
  const uint32_t lane_first = wbase + (uint32_t)win[kWinExcl][lane];
  const uint32_t lane_units = (uint32_t)win[kWinT][lane] * (uint32_t)a.Hkv;
  const uint64_t hit =
      __builtin_amdgcn_ballot_w64(lane_units > 0 && lane_first <= u0 && u0 < lane_first + lane_units);
  if (hit == 0) return;  // unreachable: u0 < total
  int L = __builtin_ctzll(hit);
  int Tl = win_at(win, kWinT, L);
  const uint32_t off = u0 - wbase - (uint32_t)win_at(win, kWinExcl, L);
  int g = (int)(off / (uint32_t)Tl);
  int b = (int)(off - (uint32_t)g * (uint32_t)Tl);
  // A short pair (at most whole_max units) is never cut: the wave whose slice
  // holds its first unit takes all of it, past the slice end if need be.
  const uint32_t whole_max = min(chunk, (uint32_t)kWholeMax);
  bool skip = b > 0 && (uint32_t)Tl <= whole_max;

  // Records of cut pairs: [nw][2][R][kRec], slot 0 for the slice's first
  // pair, slot 1 for its last; all through one buffer resource.
  const int32_t rec_range = nw * 2 * R * kRec * (int)sizeof(float);
  auto rec_off = [&](int wave, int slot, int row) {
    return (uint32_t)((((wave * 2 + slot) * R + row) * kRec) * sizeof(float));
  };
  const uint32_t dim_bytes = lc * 8 * sizeof(float);

  // Pairs this slice cuts: at most its first (record slot 0) and its last
  // (slot 1).  Their tickets are taken after the slice's last pair, so the
  // round trips of the merge protocol never stall the K/V stream.
  PairRef cut[2];
  bool has_cut[2] = {false, false};

  // Moves (r, L, g, Tl) to the next pair with work: the next KV head, else
  // the next sequence with decode blocks (loading windows as needed).
  auto next_pair = [&]() {
    if (++g < a.Hkv) return;
    g = 0;
    uint64_t more =
        __builtin_amdgcn_ballot_w64(win[kWinT][lane] > 0) & (L == 63 ? 0ull : ~0ull << (L + 1));
    while (more == 0 && r + 1 < nwin) {  // units remain past the current pair
      wbase += wtot;
      ++r;
      wtot = __builtin_amdgcn_readfirstlane(load_window(a, 64 * r, win));
      more = __builtin_amdgcn_ballot_w64(win[kWinT][lane] > 0);
    }
    L = more ? __builtin_ctzll(more) : 0;
    Tl = win_at(win, kWinT, L);
  };

  // One segment: blocks b .. b+len-1 (of the pair's Tl after `start`) from unit pos.
  struct Segment {
    PairRef pr;
    int C, start, b, len, rows;
    uint32_t pos;
  };
  auto make_segment = [&](uint32_t at, int from) {
    Segment sg;
    sg.pr.s = 64 * r + L;
    sg.pr.g = g;
    sg.pr.q0 = win_at(win, kWinQ0, L);
    sg.pr.n = win_at(win, kWinN, L);
    sg.pr.chunks = win_at(win, kWinChunks, L);
    sg.pr.Tl = Tl;
    sg.pr.p0 = wbase + (uint32_t)win_at(win, kWinExcl, L) + (uint32_t)g * (uint32_t)Tl;
    sg.C = win_at(win, kWinC, L);
    sg.start = win_at(win, kWinStart, L);
    sg.b = from;
    sg.len = (uint32_t)Tl <= whole_max ? Tl - from : (int)min((uint32_t)(Tl - from), u1 - at);
    sg.rows = sg.pr.n * a.G;
    sg.pos = at;
    return sg;
  };
  uint32_t pos = u0;
  if (skip) {  // the previous slice's wave takes this pair
    pos += (uint32_t)(Tl - b);
    if (pos >= u1) return;
    next_pair();
    b = 0;
  }
  for (;;) {
    const Segment cur = make_segment(pos, b);
    const PairRef& pr = cur.pr;
    const bool whole = cur.b == 0 && cur.len == pr.Tl;
    const int b0 = cur.start + cur.b, b1 = b0 + cur.len;
    float Mr[R], Lr[R], Or[R][8];
    attend_range<T, R, kMfma, kQuant>(a, pr.g, pr.s, pr.q0, pr.n, cur.rows, cur.C, b0, b1, Mr,
                                      Lr, Or);

    // From here lane-row lr finishes rows lr and lr + 4, lane lc dims lc*8 .. +7.
    const int slot = cur.pos == u0 ? 0 : 1;
#pragma unroll
    for (int k = 0; k < (R + 3) / 4; ++k) {
      const int row = lr + 4 * k;
      if (row >= cur.rows) continue;
      RowState st;
      pick_row<R>(Mr, Lr, Or, row, st);
      if (whole) {
        if (pr.chunks > 0) fold_prefix(pr, row, st);
        write_out(pr, row, st);
      } else {
        const uint32_t ro = rec_off(w, slot, row);
        store16_at<kSc1>(a.ws, ro + dim_bytes, rec_range,
                         __builtin_bit_cast(u32x4, f32x4{st.o[0], st.o[1], st.o[2], st.o[3]}));
        store16_at<kSc1>(a.ws, ro + dim_bytes + 16, rec_range,
                         __builtin_bit_cast(u32x4, f32x4{st.o[4], st.o[5], st.o[6], st.o[7]}));
        if (lc == 0)
          store8_at<kSc1>(a.ws, ro + 128 * sizeof(float), rec_range,
                          u32x2{__float_as_uint(st.M), __float_as_uint(st.L)});
      }
    }
    if (!whole) {
      cut[slot] = pr;
      has_cut[slot] = true;
    }
    pos = cur.pos + (uint32_t)cur.len;
    if (pos >= u1) break;
    next_pair();
    b = 0;
  }
  if (!has_cut[0] && !has_cut[1]) return;

  // A cut pair's slices are waves wf .. wl; the last of them to finish merges
  // their records.  atomicInc wraps at nseg-1 back to 0, so the counter is 0
  // again for the next call.  Records travel only through agent-coherent
  // (sc1) stores and loads, which are coherent across the XCDs' separate L2s;
  // waiting for the stores to complete before taking a ticket orders them
  // before it.  (A device-wide fence would instead write back and invalidate
  // the whole L2 of the XCD, once per wave.)
  __builtin_amdgcn_s_waitcnt(0);
  uint32_t ticket[2] = {0u, 0u};
  int nseg[2] = {0, 0};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (!has_cut[c]) continue;
    const PairRef& pr = cut[c];
    nseg[c] = (int)((pr.p0 + (uint32_t)pr.Tl - 1) / chunk - pr.p0 / chunk) + 1;
    if (lane == 0)
      ticket[c] = __builtin_amdgcn_atomic_inc32(a.counters + (size_t)pr.s * a.Hkv + pr.g,
                                                (uint32_t)(nseg[c] - 1), __ATOMIC_RELAXED,
                                                "agent");
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (!has_cut[c] || __shfl(ticket[c], 0) != (uint32_t)(nseg[c] - 1)) continue;
    const PairRef& pr = cut[c];
    const int wf = (int)(pr.p0 / chunk);
    // wave wf's record is its first pair's only if the pair starts its slice
    const int slot_f = pr.p0 == (uint32_t)wf * chunk ? 0 : 1;
    const int rows = pr.n * a.G;
#pragma unroll
    for (int k = 0; k < (R + 3) / 4; ++k) {
      const int row = lr + 4 * k;
      if (row >= rows) continue;
      RowState st;
      st.M = kNegBig;
      st.L = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) st.o[d] = 0.f;
      fold(st, nseg[c], [&](int iq, u32x2& ml, u32x4& lo, u32x4& hi) {
        const uint32_t ro = rec_off(wf + iq, iq == 0 ? slot_f : 0, row);
        ml = load8_at<kSc1>(a.ws, ro + 128 * sizeof(float), rec_range);
        lo = load16_at<kSc1>(a.ws, ro + dim_bytes, rec_range);
        hi = load16_at<kSc1>(a.ws, ro + dim_bytes + 16, rec_range);
      });
      if (pr.chunks > 0) fold_prefix(pr, row, st);
      write_out(pr, row, st);
    }
  }
}

template <typename T, int R, bool kQuant>
hipError_t launch_rows(const DecodePlan& plan, const DecodeArgs& args, hipStream_t stream) {
  // Instances of kMfmaMinRows rows and more run on the matrix cores (see attend_mfma).
  constexpr bool kMfma = R >= kMfmaMinRows;
  hipLaunchKernelGGL((decode_kernel<T, R, kMfma, kQuant>), dim3(plan.waves), dim3(64), 0, stream,
                     args);
  return hipGetLastError();
}

template <typename T, bool kQuant = false>
hipError_t launch_typed(const DecodePlan& plan, const DecodeArgs& args, hipStream_t stream) {
  switch (plan.rows) {
    case 1: return launch_rows<T, 1, kQuant>(plan, args, stream);
    case 2: return launch_rows<T, 2, kQuant>(plan, args, stream);
    case 4: return launch_rows<T, 4, kQuant>(plan, args, stream);
    default: return launch_rows<T, 8, kQuant>(plan, args, stream);
  }
}

}  // namespace

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t max_context_len, int32_t max_query_len) {
  DecodePlan plan{0, 0};
  const int32_t G = num_q_heads / num_kv_heads;
  if (G > kDecodeRows || num_seqs <= 0 || max_query_len <= 0) return plan;  // no decode rows
  int32_t need = G * max_query_len;
  if (need > kDecodeRows) need = kDecodeRows;
  int32_t rows = 1;
  while (rows < need) rows *= 2;
  plan.rows = rows;
  // A grid the chip holds at once (decode_kernel is compiled for this
  // occupancy on 256 compute units x 4 SIMDs), smaller when the batch cannot
  // give each wave kMinChunk units.  (Measured: one wave per SIMD is best on
  // the matrix cores, two on the VALU path; more only lengthens the latency
  // of every dependent load.)
  const int32_t per_simd = rows <= 2 ? 2 : 1;
  const int64_t max_blocks = (max_context_len + kBlockSize - 1) / kBlockSize;
  const int64_t bound = (int64_t)num_seqs * num_kv_heads * max_blocks;
  // The kernel's slices are at least kMinChunk units, and at least
  // min_slice(longest pair): no more waves than that leaves work for.
  int64_t min_chunk = min_slice((int)(max_blocks < INT32_MAX ? max_blocks : INT32_MAX));
  if (min_chunk < kMinChunk) min_chunk = kMinChunk;
  int64_t waves = (bound + min_chunk - 1) / min_chunk;
  if (waves > (int64_t)per_simd * 1024) waves = (int64_t)per_simd * 1024;
  if (waves < 1) waves = 1;
  plan.waves = (int32_t)waves;
  return plan;
}

namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

WorkspaceLayout workspace_layout(const DecodePlan& plan, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t max_context_len,
                                 int32_t max_query_len, size_t min_zero_bytes,
                                 bool allow_cascade) {
  WorkspaceLayout w{};
  const int32_t G = num_q_heads / num_kv_heads;
  w.prefill = (int64_t)max_query_len * G > kDecodeRows && num_seqs > 0;
  // The shared-prefix pass runs in decode-only calls (no sequence can bring
  // more than kDecodeRows rows per KV head), with two sequences and a context
  // long enough to hold kCascadeMinBlocks full blocks before the block of its
  // last key.  A call that may prefill leaves its decode sequences to read
  // shared blocks each on its own: the pass and its plan would cost such a
  // call two launches for the few decode sequences it holds.
  w.cascade = allow_cascade && plan.rows > 0 && !w.prefill && num_seqs >= 2 &&
              max_context_len > kCascadeMinBlocks * kBlockSize;
  if (w.cascade) {
    // Work items: at most num_seqs / 2 groups, each with at most as many
    // chunks as the longest shareable range allows.
    const int64_t cap = (max_context_len - 1) / kBlockSize;
    const int64_t tiles = (cap * kBlockSize + 63) / 64;
    int64_t chunks = tiles / kChunkTiles;
    if (chunks < 1) chunks = 1;
    if (chunks > kPrefixChunks) chunks = kPrefixChunks;
    w.max_items = (int32_t)((num_seqs / 2) * chunks * num_kv_heads);
  }
  // One wave takes the whole batch: no pair is ever cut.
  const bool split = plan.rows > 0 && plan.waves > 1;
  // The zero region comes first, at fixed offsets, so that every call finds
  // its item count and counters where earlier calls left them at zero.
  // Its size depends on num_seqs * num_kv_heads alone (the item count's 256
  // B and the counters), whichever regions follow, so that a workspace serves
  // later calls of any kind with at most as many pairs without a new
  // zero-fill (a prefill's work queues never land where a later call looks
  // for its item count).
  w.item_count = 0;
  w.counters = 256;
  size_t zero = 0;
  if (w.cascade || split || w.prefill)
    zero = 256 + align256((size_t)num_seqs * num_kv_heads * sizeof(uint32_t));
  if (zero < min_zero_bytes) zero = align256(min_zero_bytes);
  w.zero_bytes = zero;
  size_t off = zero;
  w.starts = off;
  if (w.cascade) off += align256((size_t)num_seqs * 2 * sizeof(int32_t));
  w.items = off;
  if (w.cascade) off += align256((size_t)w.max_items * 8 * sizeof(int32_t));
  w.prefix = off;
  if (w.cascade)
    off += align256((size_t)num_seqs * num_q_heads * kPrefixChunks * kRecFloats * sizeof(float));
  w.records = off;
  if (split) off += (size_t)plan.waves * 2 * plan.rows * kRecFloats * sizeof(float);
  w.queue = off;
  if (w.prefill) off += 256;
  w.order = off;
  if (w.prefill) off += align256((size_t)num_seqs * sizeof(int32_t));
  w.total = off;
  return w;
}

hipError_t launch_decode(bool is_bf16, const DecodePlan& plan, const WorkspaceLayout& ws,
                         void* out, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, const int32_t* query_start_loc,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         float scale, void* workspace, hipStream_t stream, bool rank_prefill) {
  char* base = static_cast<char*>(workspace);
  DecodeArgs args;
  args.order = rank_prefill ? reinterpret_cast<int32_t*>(base + ws.order) : nullptr;
  args.queue = rank_prefill ? reinterpret_cast<int32_t*>(base + ws.queue) : nullptr;
  args.q = static_cast<const uint16_t*>(q);
  args.k_pool = static_cast<const uint16_t*>(k_pool);
  args.v_pool = static_cast<const uint16_t*>(v_pool);
  args.block_tables = block_tables;
  args.context_lens = context_lens;
  args.qsl = query_start_loc;
  args.out = static_cast<uint16_t*>(out);
  args.counters = base ? reinterpret_cast<uint32_t*>(base + ws.counters) : nullptr;
  args.ws = base ? reinterpret_cast<float*>(base + ws.records) : nullptr;
  args.starts = ws.cascade ? reinterpret_cast<const int32_t*>(base + ws.starts) : nullptr;
  args.prefix_rec = ws.cascade ? reinterpret_cast<const float*>(base + ws.prefix) : nullptr;
  args.item_count = ws.cascade ? reinterpret_cast<int32_t*>(base + ws.item_count) : nullptr;
  args.max_blocks = max_blocks_per_seq;
  args.Hq = num_q_heads;
  args.Hkv = num_kv_heads;
  args.G = num_q_heads / num_kv_heads;
  args.S = num_seqs;
  args.scale_log2 = scale * kLog2e;
  args.qpool = nullptr;
  args.page_tables = nullptr;
  args.quant_lens = nullptr;
  args.max_pages = 0;
  return is_bf16 ? launch_typed<bf16>(plan, args, stream) : launch_typed<f16>(plan, args, stream);
}

hipError_t launch_decode_quant(bool is_bf16, const DecodePlan& plan, const WorkspaceLayout& ws,
                               void* out, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               float scale, const QuantArgs& qa, void* workspace,
                               hipStream_t stream) {
  char* base = static_cast<char*>(workspace);
  DecodeArgs args;
  args.q = static_cast<const uint16_t*>(q);
  args.k_pool = static_cast<const uint16_t*>(k_pool);
  args.v_pool = static_cast<const uint16_t*>(v_pool);
  args.block_tables = block_tables;
  args.context_lens = context_lens;
  args.qsl = query_start_loc;
  args.out = static_cast<uint16_t*>(out);
  args.counters = base ? reinterpret_cast<uint32_t*>(base + ws.counters) : nullptr;
  args.ws = base ? reinterpret_cast<float*>(base + ws.records) : nullptr;
  args.starts = nullptr;
  args.prefix_rec = nullptr;
  args.item_count = nullptr;
  args.order = nullptr;
  args.queue = nullptr;
  args.qpool = qa.qpool;
  args.page_tables = qa.page_tables;
  args.quant_lens = qa.quant_lens;
  args.max_pages = qa.max_pages;
  args.max_blocks = max_blocks_per_seq;
  args.Hq = num_q_heads;
  args.Hkv = num_kv_heads;
  args.G = num_q_heads / num_kv_heads;
  args.S = num_seqs;
  args.scale_log2 = scale * kLog2e;
  return is_bf16 ? launch_typed<bf16, true>(plan, args, stream)
                 : launch_typed<f16, true>(plan, args, stream);
}

}  // namespace pa
