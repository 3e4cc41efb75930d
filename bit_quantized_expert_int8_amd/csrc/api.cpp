// Error reporting, record layout and version: the host-only part of the C ABI.
#include <stdarg.h>
#include <stdio.h>
#include <string>

#include "common.h"

namespace moeq4 {

static thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

bool record_offsets(int32_t d, int32_t F, moe_dtype sb, RecordOffsets* out) {
  if (d <= 0 || F <= 0 || d % 64 || F % 64 || (sb != MOE_F32 && sb != MOE_BF16)) return false;
  const size_t sbw = sb == MOE_BF16 ? 2 : 4;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t D = (size_t)d, FF = (size_t)F;
  out->gate_up_q = 0;
  out->gate_up_sb = up(2 * FF * D / 2);
  out->down_q = up(out->gate_up_sb + 2 * FF * (D / 64) * 2 * sbw);
  out->down_sb = up(out->down_q + D * FF / 2);
  out->total = up(out->down_sb + D * (FF / 64) * 2 * sbw);
  return true;
}

}  // namespace moeq4

using namespace moeq4;

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_version(void) { return "moeq4 0.1 gfx950"; }

size_t moe_record_bytes(int32_t d, int32_t F, moe_dtype sb_dtype) {
  RecordOffsets o;
  return record_offsets(d, F, sb_dtype, &o) ? o.total : 0;
}

moe_status moe_record_layout(int32_t d, int32_t F, moe_dtype sb_dtype, size_t offsets[4]) {
  RecordOffsets o;
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "moe_record_layout: offsets is NULL");
  if (!record_offsets(d, F, sb_dtype, &o))
    return fail(MOE_ERR_INVALID_ARG, "moe_record_layout: d=%d F=%d must be positive multiples of 64", d, F);
  offsets[0] = o.gate_up_q;
  offsets[1] = o.gate_up_sb;
  offsets[2] = o.down_q;
  offsets[3] = o.down_sb;
  return MOE_OK;
}

}  // extern "C"
