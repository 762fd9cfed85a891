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

}  // namespace tilemix
