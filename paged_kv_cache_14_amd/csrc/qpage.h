// Layout of one quantized KV page of one KV head: 128 tokens x 128
// channels, keys per channel and values per token at 2 bits, 16 promoted key
// channels at 4 (KV-cache textbook ch.22, the Kitty passage).  A pool of
// quantized pages is [num_pages][num_kv_heads][kQPageBytes] bytes.
//
// The code fields follow the matrix-core decode's operand layout.  A page is
// 4 steps of 32 tokens (two 16-token blocks); in a step, decode lane
// l = 16q + j (q = l / 16, j = l % 16) owns, in its 16 bytes (4 words), the
// 16-bit operands of v_mfma_f32_16x16x32_f16 it needs, as f16 pairs: bit
// pair i (i = 0..7) of a word holds one code at bits 2i and the next at bits
// 16 + 2i, so that (word >> 2i) & 0x00030003 is the pair.
//   kQKLo     [4 steps][64 lanes][4 words]: low 2 bits of the key codes.
//             Word w: half H = w / 2, channel block m = 2(w % 2) + i / 4,
//             pair p = i % 4; key kk = 8(j / 4) + 4H + j % 4 of the step;
//             channels 32m + 8q + 2p (bits 2i) and + 1 (bits 16 + 2i).
//   kQKHi     [4 steps][32 lanes (q < 2)][1 word]: high 2 bits of the
//             promoted key channels: bit pair i = 4H + p holds promoted
//             slots 8q + 2p and 8q + 2p + 1 of key kk(H, j).
//   kQKScale  [128] float: key step per channel (span / 15 promoted, / 3 not)
//   kQKMin    [128] float: key minimum per channel
//   kQBoostList [16] uint8: the promoted channels, ascending (64 B kept)
//   kQVLo     [4 steps][64 lanes][4 words]: value codes.  Word w: dim tile
//             t = 2w + i / 4, pair p = i % 4; dim 16t + j; keys 8q + 2p
//             (bits 2i) and 8q + 2p + 1 (bits 16 + 2i) of the step.
//   kQVScale  [128] float: value step per token
//   kQVMin    [128] float: value minimum per token
#pragma once

namespace pa {

constexpr int kQPageTokens = 128;
constexpr int kQPageBlocks = kQPageTokens / 16;
constexpr int kQBoost = 16;
constexpr int kQKLo = 0;
constexpr int kQKHi = kQKLo + 4096;
constexpr int kQKScale = kQKHi + 512;
constexpr int kQKMin = kQKScale + 512;
constexpr int kQBoostList = kQKMin + 512;
constexpr int kQVLo = kQBoostList + 64;
constexpr int kQVScale = kQVLo + 4096;
constexpr int kQVMin = kQVScale + 512;
constexpr int kQPageBytes = kQVMin + 512;  // 10816

}  // namespace pa
