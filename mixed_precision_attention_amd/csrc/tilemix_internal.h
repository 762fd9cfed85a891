// Internal layout of the TileMix work plan, shared by the host planner and
// the device kernels of libtilemix.  Not part of the public ABI.
#pragma once

#include <stdint.h>

namespace tilemix {

constexpr int32_t kPlanMagic = 0x544D5850;  // "TMXP"
constexpr int32_t kPlanVersion = 3;

// Header fields (int32 indices into the plan).
enum PlanField : int {
  kMagic = 0,
  kVersion = 1,
  kBatch = 2,
  kHq = 3,
  kHkv = 4,
  kHeadDim = 5,
  kTotalTokens = 6,
  kTotalQTiles = 7,
  kTotalKTiles = 8,
  kNumItems = 9,      // work units in the launch order, padding included
  kSeqOff = 10,       // offset of the per-sequence table
  kItemOff = 11,      // offset of the work-unit list
  kPlanDies = 12,     // dies the list is interleaved over
  kMaxTm = 13,        // largest Tm of any sequence
  kPlanHash = 14,     // checksum (FNV-1a over words, 4 streams) of every other field and the body
  kHeaderLen = 16
};

// Per-sequence record (kSeqStride int32 each).
enum SeqField : int {
  kSeqStart = 0,   // first packed token
  kSeqLen = 1,     // L
  kSeqQtOff = 2,   // first global query tile
  kSeqKtOff = 3,   // first global key tile
  kSeqG = 4,       // grouping factor
  kSeqTm = 5,
  kSeqTn = 6,
  kSeqStride = 8
};

// Work unit: two int32, {seq (or -1 for padding), (head << 16) | row}.
constexpr int kItemStride = 2;

constexpr int kBlockM = 128;
constexpr int kBlockN = 64;
constexpr int kWordBits = 64;

}  // namespace tilemix
