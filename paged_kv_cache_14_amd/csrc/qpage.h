// Layout of one quantized KV page of one KV head: 128 tokens x 128
// channels, keys per channel and values per token at 2 bits, 16 promoted key
// channels at 4 (KV-cache textbook ch.22, the Kitty passage).  A pool of
// quantized pages is [num_pages][num_kv_heads][kQPageBytes] bytes.
//
// The code fields follow the decode's lane order: decode lane l holds
// channels 8j .. 8j+7 (j = l % 16) of tokens 4i + r (r = l / 16, i = 0..3)
// of each 16-token block, so each lane's codes for a block are one 8-byte
// field and a wave's fields for a block are 512 contiguous bytes.
//   kQKLo     [8 blocks][16 j][4 r] x 8 B: low 2 bits of every key code;
//             token i in bits 16i..16i+15, channel 8j + e at bits 2e.
//   kQKHi     [16 slots][4 r][8 blocks] x 1 B: high 2 bits of promoted key
//             channel boost[slot]; token 4i + r of the block in bits 2i.
//   kQKScale  [128] float: key step per channel (span / 15 promoted, / 3 not)
//   kQKMin    [128] float: key minimum per channel
//   kQBoostList [16] uint8: the promoted channels, ascending (64 B kept)
//   kQVLo     as kQKLo, the value codes (2 bits)
//   kQVScale  [8 blocks][4 r][4 i] float: value step of token 4i + r
//   kQVMin    same order: value minimum of that token
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
