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
constexpr int64_t kDecodeItemsTarget = 1024; // items x KV heads the chunk size aims for (fewer, longer items pay fewer workgroup start-ups)
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
