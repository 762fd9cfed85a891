// Host helpers shared by the two translation units of libtilemix.
#pragma once

#include <stdint.h>

namespace tilemix {

struct SeqGeo {
  int64_t L = 0, Tm = 0, Tn = 0, g = 1;
  int64_t last_tile(int64_t r) const;   // last key tile holding a legal pair of row r
  int64_t last_group(int64_t r) const;  // D(r)
};

SeqGeo geometry(int64_t L);

int fail(int code, const char* fmt, ...);
void clear_error();
const char* last_error();
bool aligned16(const void* p);
int check_cu_seqlens(const int32_t* cu, int32_t batch);
int check_plan(const int32_t* plan_h);
// Length in int32 of a plan whose header passed check_plan.
int64_t plan_length(const int32_t* plan_h);
// Checksum of a plan's header (its hash field counted as 0) and body: four
// interleaved word-wise FNV-1a (32-bit) streams, folded, xor the length.
uint32_t plan_hash(const int32_t* plan_h);
// check_plan on the host copy, then the device copy's pointer; a build with
// TILEMIX_DEBUG_PLAN also reads back the device copy's header and requires it
// to equal the host copy's (hash included).
int check_plans(const int32_t* plan_h, const int32_t* plan_d);

}  // namespace tilemix
