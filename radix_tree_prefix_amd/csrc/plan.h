// Constants and layouts shared by the decode-plan builder and the decode kernel.
#pragma once

#include <cstdint>

#include "rs.h"

namespace rs {

constexpr int32_t kPlanMagic = 0x52535031;   // "RSP1"
constexpr int32_t kPlanHeaderWords = 16;
constexpr int32_t kItemWords = 8;            // k0, k1, rep_row, n_req, req_off, -, -, -
constexpr int32_t kItemReqWords = 4;         // request, partial index, partials of the request, -
constexpr int32_t kMaxRowsPerItem = 128;     // 4 waves x 32 query rows
constexpr int32_t kFlatChunk = 256;          // keys per item in the flat (plan-less) mode
// items x KV heads the chunk size aims for: three quarters of the 512 decode workgroups the
// chip holds at once (two per CU), so every item starts in the first round and fewer, longer
// items pay fewer start-ups.  Measured against 1024 / 512 / 256: mixed batch 661 vs 671 / 661 /
// 663 us, preamble agent 25.4 vs 27.3 / 26.8 / 27.4 us, tree of thought 63.2 vs 71.4 / 63.3 /
// 71.2 us.
constexpr int64_t kDecodeItemsTarget = 384;
constexpr int64_t kMinChunk = 256;           // >= 4 tiles per item (shorter ones measured slower on the small batches)
constexpr int64_t kMaxChunk = 8192;
constexpr int32_t kChunkAlign = 64;          // item key ranges start at multiples of this (whole decode tiles)

// Decode workspace: o partials float [Hkv][P][G][D], lse partials float [Hkv][P][G];
// each region 256-byte aligned.
struct WsLayout {
  int64_t o_off, lse_off, bytes;
};
WsLayout ws_layout(int64_t n_partials, int32_t B, int32_t Hq, int32_t Hkv, int32_t D);
const rs_plan_info_t* plan_info(const rs_plan* p);

// Word offsets of the plan image's arrays (items, item_req, part_ptr).
struct PlanOffsets {
  int32_t items, item_req, part_ptr;
};
PlanOffsets plan_offsets(const rs_plan* p);

}  // namespace rs
